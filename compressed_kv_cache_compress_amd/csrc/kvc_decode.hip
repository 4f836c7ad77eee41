// kvc_decode.hip -- gfx950 decode attention over compressed KV segments
// (MosaicKV review page, Fig. 6 caption: PackedAttention over the packed KV
// format).
//
// Work split: one wave per (stream, split); a split is a contiguous range of
// the stream's descriptors.  Four independent waves share a workgroup only to
// share one LDS table.  Each wave walks its descriptors in chunks of up to 16
// kept tokens (fewer for rows wider than 96 channels):
//   * the next chunk's K and V bytes (masks + compact values) are loaded into
//     registers while the current chunk is computed, then written to LDS;
//   * every kept vector is expanded from (bitmask, compact bf16 values) to a
//     dense 128-channel row, one mask byte (8 channels) per lane and step,
//     one nibble (4 channels) at a time: the nibble's candidate values are
//     the 4 compact elements starting at its rank (an 8-byte window, shifted
//     by one element when the rank is odd), and one v_perm_b32 per output
//     dword places them (or zero) using a 16-entry selector table indexed by
//     the nibble;
//   * staged rows are padded by 16 bytes so that the 16 tokens of a chunk
//     start on different LDS banks;
//   * q.k of the 16 tokens and p.v run on MFMA (bf16 inputs, fp32
//     accumulation); the softmax is online, in base 2, with DPP row
//     reductions.
// A second kernel merges the splits (log-sum-exp) and rounds to bf16.
//
// MFMA row mapping: q head h of the group is A-row 4*(h & 3) + (h >> 2), so
// in the 16x16 accumulator layout (lane l, item j <-> row 4*(l>>4)+j, column
// l&15) lane l's item j belongs to head 4*j+(l>>4) and to token/channel l&15;
// for G <= 4 every head lives in item 0 of its own 16-lane row.  For G <= 4
// the p.v product uses the 16-block 4x4x4 MFMA instead (block b = lanes
// 4b..4b+3; A[i][k] at lane 4b+i item k, B[k][j] at lane 4b+j item k, D[i][j]
// at lane 4b+j item i): head i x channel (64*half + lane) accumulates over 4
// tokens per instruction, so the output needs 8 instead of 32 registers.  Its
// B operand (4 tokens x 1 channel per lane) comes from the row-major dense V
// tile through ds_read_b64_tr_b16: within each 16-lane group, element r of
// lane i is element (i & 3) of the 8 bytes read by lane 4r + (i >> 2), so lane
// l reads row 4*sg + ((l & 15) >> 2), channels 64*half + 16*(l >> 4) + 4*(l & 3).
#include <hip/hip_runtime.h>
#include <cstdint>

#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) const uint32_t lds_u32_t;
typedef __attribute__((address_space(1))) const u32x4_t glb_u32x4_t;

// LDS byte offset of a pointer into shared memory, and back.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_u32_t*)p;
}
__device__ __forceinline__ const lds_u32_t* lds_ptr(uint32_t off) {
  return (const lds_u32_t*)(uintptr_t)off;
}

constexpr int CT = 16;  // MFMA columns: at most this many kept tokens per chunk
#ifndef KVC_DECODE_SLOTS
#define KVC_DECODE_SLOTS 3
#endif
// uint4 prefetch slots per lane and side: a chunk side (masks + values) is at
// most 64 * NPF slots of 16 bytes.
constexpr int NPF = KVC_DECODE_SLOTS;
// Tokens per chunk for c kept channels: at most CT, at most what the prefetch
// slots hold, and at most 3584 staged bytes (16 tokens up to c = 96), so that
// wide rows do not set the staging size.  Narrow rows get 16 tokens; dense
// rows 12.
constexpr int slots_per_token(int c) { return (c < D ? 1 : 0) + c / 8; }
constexpr int staged_per_token(int c) { return (c < D ? 16 : 0) + 2 * c + 16; }
constexpr int cmin(int x, int y) { return x < y ? x : y; }
constexpr int cmax(int x, int y) { return x > y ? x : y; }
constexpr int chunk_tokens(int c) {
  return cmin(CT, cmin(64 * NPF / slots_per_token(c), 3584 / staged_per_token(c)));
}
constexpr int stage_bytes() {
  int m = 0;
  for (int c = 8; c <= D; c += 8) m = cmax(m, chunk_tokens(c) * staged_per_token(c));
  return m + 32;  // + pad: a window may read 12 bytes past a row's last element
}
// Staging bytes of one side of a chunk: [masks 16 * nt][rows (2c + 16) * nt].
constexpr int STAGE = (stage_bytes() + 15) / 16 * 16;
constexpr float RESCALE_SLACK = 8.0f;             // log2 units the running max may lag
constexpr int VT_STRIDE = 20;                     // u16 per channel row of the transposed V tile (G > 4)
constexpr int VR_STRIDE = 136;                    // u16 per token row of the row-major V tile (G <= 4)
constexpr int WAVES = 4;
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
  float sl2;  // scale * log2(e)
};

// Per-wave LDS.  The loop is software-pipelined: while the K side of chunk
// i+1 is computed, the V side of chunk i is, so V stages and probabilities
// are double-buffered.  A V stage's dense tile is written from the registers
// its own reads produced, so the two share storage.
// JG == 1: row-major dense V tile [token][VR_STRIDE]; otherwise transposed
// [channel][VT_STRIDE].  Either is written over the V stage it is expanded from.
template <int JG>
struct VStage {
  static constexpr int BYTES = cmax(STAGE, JG == 1 ? CT * VR_STRIDE * 2 : D * VT_STRIDE * 2);
  union {
    u32x4_t v[BYTES / 16];
    uint16_t vt[BYTES / 2];
  };
};
template <int JG>
struct WaveLds {
  u32x4_t k[STAGE / 16];
  VStage<JG> vs[2];               // chunk i's V side and chunk i+1's, alternating
  uint16_t pl[2][4 * JG * CT];    // probabilities, [head][token], alternating
};

static_assert(chunk_tokens(64) == CT && chunk_tokens(D) >= 12, "stage sizing");


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
    e.tl[kk] = lut[mb & 0xFu];
    e.th[kk] = lut[mb >> 4];
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

// One chunk to stream: K part and V part each = [masks 16*nt][values 2*c*nt]
// in global memory.  Uniform bases: the value stream of a side is addressed
// as val + 16*j for stream slot j >= nm (val already offset by -16*nm).
struct Chunk {
  const uint8_t* kmask;
  const uint8_t* kval;
  const uint8_t* vmask;
  const uint8_t* vval;
  int nt, c, nm, n16;
  uint32_t magic;  // ceil(2^20 / (c/8)): value slot -> row by multiply-shift
  bool valid;
};

// The next chunk's bytes, one uint4 of K and one of V per slot and lane.
struct Regs {
  u32x4_t k[NPF], v[NPF];
};

template <int I>
__device__ __forceinline__ void prefetch_slot(const Chunk& ch, int lane, Regs& r) {
  const int j = lane + 64 * I;
  if (j < ch.n16) {
    // the packed buffer is device (global) memory; an unsigned 32-bit
    // offset on a scalar base is the load's native addressing form
    const uint32_t off = 16u * (uint32_t)j;
    if (I == 0 && j < ch.nm) {
      r.k[I] = *(glb_u32x4_t*)(ch.kmask + off);
      r.v[I] = *(glb_u32x4_t*)(ch.vmask + off);
    } else {
      r.k[I] = *(glb_u32x4_t*)(ch.kval + off);
      r.v[I] = *(glb_u32x4_t*)(ch.vval + off);
    }
  }
}

__device__ __forceinline__ void prefetch(const Chunk& ch, int lane, Regs& r) {
  if (!ch.valid) return;
  prefetch_slot<0>(ch, lane, r);
  prefetch_slot<1>(ch, lane, r);
  prefetch_slot<2>(ch, lane, r);
  if constexpr (NPF > 3) prefetch_slot<3>(ch, lane, r);
}

// Slot j of the [masks | values] stream goes to LDS slot j (masks) or, for
// value slot v = j - nm, to nm + v + v / (c/8): one 16-byte pad per row.
template <int I>
__device__ __forceinline__ void commit_slot(const Chunk& ch, int lane, const Regs& r, u32x4_t* sk,
                                            u32x4_t* sv) {
  const int j = lane + 64 * I;
  if (j < ch.n16) {
    const uint32_t v = (uint32_t)(j - ch.nm);
    const int dst = (I == 0 && j < ch.nm) ? j : j + (int)(__umul24(v, ch.magic) >> 20);
    sk[dst] = r.k[I];
    sv[dst] = r.v[I];
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

__device__ __forceinline__ void fetch_descs(Cursor& cu, int lane) {
  cu.base = cu.di;
  const int i = min(cu.di + lane, cu.d1 - 1);
  const u32x4_t d = *reinterpret_cast<const u32x4_t*>(cu.dl + i);
  cu.w0 = d[0];
  cu.w1 = d[1];
  cu.w2 = d[2];
  // per-descriptor chunk geometry, computed once per 64 descriptors so that
  // the chunk loop reads it with readlane instead of a memory lookup; a
  // paged descriptor (flags bit2) also carries log2(seg_tokens) + 1, the
  // token count its parts are laid out for
  const int c = (int)(d[2] >> 16) & ~7;
  const int cc = c < 8 ? 8 : (c > D ? D : c);
  const uint32_t cap = d[3] >> 16;
  const uint32_t page = ((d[3] >> 8) & KVC_DESC_PAGED) && cap ? 32u - __clz(cap) : 0u;
  cu.w3 = (uint32_t)chunk_tokens(cc) | (row_magic(cc >> 3) << 5) | (page << 26);
}

// Chunks of descriptor i of a stream's list (0 past nd): ceil(T / ct) with
// ct = 12 to 16 tokens per chunk.  T / ct is a multiple of 1/ct >= 1/16 apart
// from the next integer, so adding 31/32 to the product with the approximate
// reciprocal and truncating gives the exact ceiling.  (The count only
// balances the splits; any count gives the same results.)
__device__ __forceinline__ uint32_t desc_chunks(const kvc_seg_desc* dl, int i, int nd) {
  if (i >= nd) return 0u;
  const uint32_t tc = reinterpret_cast<const uint32_t*>(dl + i)[2];
  const uint32_t T = tc & 0xFFFFu;
  const int c = (int)(tc >> 16) & ~7;
  const float ct = (float)chunk_tokens(c < 8 ? 8 : (c > D ? D : c));
  return (uint32_t)((float)T * __builtin_amdgcn_rcpf(ct) + 0.96875f);
}
// inclusive sum over the 64 lanes: rows by row_shr, then the row broadcasts
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);
  return x;
}

// Descriptor range [di, d1) of split sp of a stream with nd descriptors.
// With more descriptors than splits and at most 256 of them, splits take
// equal shares of chunks: descriptor i goes to split floor(E_i * splits / W),
// with E_i the chunks of the descriptors before i and W all chunks of the
// stream.  That index never decreases with i, so every split takes a
// contiguous run (possibly empty).  Few descriptors per split of different
// sizes (a dense prompt page is 22 chunks, a Kara event segment 1) leave one
// wave with most of a stream's work otherwise.  Over longer lists equal
// descriptor counts balance well enough: at 1024 descriptors per stream the
// scan cost more than it saved.
__device__ __forceinline__ void split_range(const kvc_seg_desc* dl, int nd, int splits, int sp,
                                            int lane, int& di, int& d1) {
  di = (int)(((int64_t)sp * nd) / splits);
  d1 = (int)(((int64_t)(sp + 1) * nd) / splits);
  if (nd <= splits || nd > 256) return;
  uint32_t part = 0;
  for (int i = lane; i < nd; i += 64) part += desc_chunks(dl, i, nd);
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_u32(part), 63);
  if (total == 0) return;
  // split(i) < t  <=>  E_i * splits < t * W
  const uint32_t lo = (uint32_t)sp * total, hi = (uint32_t)(sp + 1) * total;
  uint32_t carry = 0;
  int nlo = 0, nhi = 0;
  for (int i0 = 0; i0 < nd; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t w = desc_chunks(dl, i, nd);
    const uint32_t x = wave_incl_scan_u32(w);
    const uint32_t e = (carry + x - w) * (uint32_t)splits;
    carry += (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
    nlo += __popcll(__ballot(i < nd && e < lo));
    nhi += __popcll(__ballot(i < nd && e < hi));
  }
  di = nlo;
  d1 = sp == splits - 1 ? nd : nhi;
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
      ++cu.di;
      if (T > 0) {
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
        cu.T = T;
        cu.c = c;
        cu.t0 = 0;
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
  __shared__ uint2 lut[16];
  __shared__ u32x4_t zrow[1];
  __shared__ WaveLds<JG> wl[WAVES];
  const int tid = threadIdx.x;
  static_assert(64 * WAVES == 256, "one selector entry per thread");
  if (tid < 16) {
    uint32_t lo[2];
    build_lut_entry((uint32_t)tid, lo);
    lut[tid] = make_uint2(lo[0], lo[1]);
    if (tid == 0) zrow[0] = u32x4_t{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  const int lane = tid & 63, wv = tid >> 6;
  const int item = blockIdx.x * WAVES + wv;
  if (item >= a.items) return;
  const int s = item / a.splits, sp = item - s * a.splits;
  const int grp = lane >> 4, col = lane & 15;
  const int b = s / a.hkv, h = s - b * a.hkv;
  WaveLds<JG>& L = wl[wv];
  for (int i = lane; i < 2 * 4 * JG * CT; i += 64) (&L.pl[0][0])[i] = 0;

  // A operand of the score MFMA: row col holds head hh (zero if none); with
  // QLO and JG == 1, row 4h + 1 holds the low part of head h
  constexpr bool LO_ROWS = QLO && JG == 1;
  const bool lo_row = LO_ROWS && (col & 3) == 1 && (col >> 2) < a.G;
  const int hh = lo_row ? (col >> 2) : 4 * (col & 3) + (col >> 2);
  const bool hh_ok = lo_row || hh < a.G;
  const uint16_t* qh = (lo_row ? a.q_lo : a.q) +
                       ((uint64_t)(b * a.hq + h * a.G + (hh_ok ? hh : 0))) * D;
  bf16x8_t qa[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (hh_ok) v = *reinterpret_cast<const u32x4_t*>(qh + 8 * (4 * kk + grp));
    qa[kk] = __builtin_bit_cast(bf16x8_t, v);
  }
  bf16x8_t qlo[QLO && !LO_ROWS ? 4 : 1];
  if constexpr (QLO && !LO_ROWS) {
    const uint16_t* ql = a.q_lo + ((uint64_t)(b * a.hq + h * a.G + (hh_ok ? hh : 0))) * D;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (hh_ok) v = *reinterpret_cast<const u32x4_t*>(ql + 8 * (4 * kk + grp));
      qlo[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // JG == 1: O4[half][item i] = head i, channel 64*half + lane (4x4x4 MFMA);
  // otherwise O[nn] is the 16x16 tile of channels 16*nn .. +15
  constexpr int NO = JG == 1 ? 2 : 8;
  f32x4_t O[NO];
#pragma unroll
  for (int nn = 0; nn < NO; ++nn) O[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
  split_range(cu.dl, nd, a.splits, sp, lane, cu.di, cu.d1);
  cu.T = 0;
  cu.c = 0;
  cu.t0 = 0;
  if (cu.di < cu.d1) fetch_descs(cu, lane);

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
  // V side of a chunk staged in L.vs[vb]: dense V tile (over the stage),
  // then O += P V with the probabilities in L.pl[vb].
  auto v_side = [&](const Chunk& ch, int vb) {
    VStage<JG>& S = L.vs[vb];
    if (JG == 1) {
      // row-major dense tile [token][channel], row stride VR_STRIDE
      static_assert(2 * VR_STRIDE == 2 * D + 16, "dense staged rows are the tile rows");
      if (ch.c == D) {
        // dense rows are staged exactly as the tile; rows past the chunk may
        // hold older data (their probabilities are 0, but 0 * NaN is NaN)
        const int nz = (CT - ch.nt) * (VR_STRIDE / 8);
        for (int i = lane; i < nz; i += 64) {
          const u32x4_t z = {0u, 0u, 0u, 0u};
          S.v[ch.nt * (VR_STRIDE / 8) + i] = z;
        }
      } else {
        u32x4_t vv[4];
        expand_side<true>(reinterpret_cast<const uint8_t*>(S.v), col, grp, ch.nt, ch.c, lut, zrow,
                          vv);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          *reinterpret_cast<u32x4_t*>(S.vt + col * VR_STRIDE + 8 * (4 * kk + grp)) = vv[kk];
      }
      const int trow = (lane & 15) >> 2, tcol = 16 * (lane >> 4) + 4 * (lane & 3);
#pragma unroll
      for (int sg = 0; sg < CT / 4; ++sg) {
        // A: head (lane & 3) x tokens 4sg..4sg+3; B: tokens x channel 64*hf + lane
        const s16x4_t pa = *reinterpret_cast<const s16x4_t*>(L.pl[vb] + (lane & 3) * CT + 4 * sg);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint16_t* src = S.vt + (4 * sg + trow) * VR_STRIDE + 64 * hf + tcol;
          const s16x4_t w = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)src);
          O[hf] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pa, w, O[hf], 0, 0, 0);
        }
      }
    } else {
      // transposed dense tile [channel][token]
      u32x4_t vv[4];
      const uint8_t* sv8 = reinterpret_cast<const uint8_t*>(S.v);
      if (ch.c < D)
        expand_side<true>(sv8, col, grp, ch.nt, ch.c, lut, zrow, vv);
      else
        expand_side<false>(sv8, col, grp, ch.nt, ch.c, lut, zrow, vv);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint16_t* dst = S.vt + (8 * (4 * kk + grp)) * VT_STRIDE + col;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[(2 * i) * VT_STRIDE] = (uint16_t)(vv[kk][i] & 0xFFFFu);
          dst[(2 * i + 1) * VT_STRIDE] = (uint16_t)(vv[kk][i] >> 16);
        }
      }
      s16x4_t pa = {0, 0, 0, 0};
      if (hh_ok) pa = *reinterpret_cast<const s16x4_t*>(L.pl[vb] + hh * CT + 4 * grp);
#pragma unroll
      for (int nn = 0; nn < NO; ++nn) {
        const s16x4_t w = *reinterpret_cast<const s16x4_t*>(S.vt + (16 * nn + col) * VT_STRIDE + 4 * grp);
        O[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, w, O[nn], 0, 0, 0);
      }
    }
  };
  auto rescale = [&](const float* alpha) {
    if (JG == 1) {
      // every lane holds all four heads: alpha of head i sits in row i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha[0]), 16 * i));
        O[0][i] *= ai;
        O[1][i] *= ai;
      }
    } else {
#pragma unroll
      for (int j = 0; j < JG; ++j)
#pragma unroll
        for (int nn = 0; nn < NO; ++nn) O[nn][j] *= alpha[j];
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
    // iteration: stage chunk i+1, load chunk i+2, K side of i+1, V side of i
    while (nxt.valid) {
        commit(nxt, lane, rg, L.k, L.vs[vb ^ 1].v);
      const Chunk far = next_chunk(cu, lane);
      prefetch(far, lane, rg);
        const bool resc = k_side(nxt, vb ^ 1, alpha);
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
#pragma unroll
  for (int j = 0; j < JG; ++j) {
    const int hd = 4 * j + grp;
    if (hd < a.G && col == 0) {
      const uint64_t pi = (uint64_t)(b * a.hq + h * a.G + hd) * a.splits + sp;
      a.part_ml[2 * pi] = m_run[j];
      a.part_ml[2 * pi + 1] = l_run[j];
    }
  }
  if (JG == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < a.G) {
        const uint64_t pi = (uint64_t)(b * a.hq + h * a.G + i) * a.splits + sp;
        a.part_acc[pi * D + lane] = O[0][i];
        a.part_acc[pi * D + 64 + lane] = O[1][i];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < JG; ++j) {
      const int hd = 4 * j + grp;
      if (hd < a.G) {
        const uint64_t pi = (uint64_t)(b * a.hq + h * a.G + hd) * a.splits + sp;
#pragma unroll
        for (int nn = 0; nn < NO; ++nn) a.part_acc[pi * D + 16 * nn + col] = O[nn][j];
      }
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
  for (int sp = g; sp < splits; sp += RG) M = fmaxf(M, ml[2 * sp]);
  float L = 0.0f, acc = 0.0f;
  if (M != -INFINITY) {
    for (int sp = g; sp < splits; sp += RG) {
      const float w = exp2f(ml[2 * sp] - M);
      L += ml[2 * sp + 1] * w;
      acc += acc_row[(uint64_t)sp * D + c0 + c] * w;
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

// Rotated cache: the same merge over all 128 channels (grid batch*n_q_heads,
// four slices of RC channels per block, one after the other), then
// out = R_V o' (o' = the merged output in the rotated basis, fp32) before the
// single bf16 rounding.  R_V of row r's stream is read row by row.
template <int RG, int RC>
__global__ __launch_bounds__(RG * RC) void k_decode_reduce_rot(const float* __restrict__ part_ml,
                                                             const float* __restrict__ part_acc,
                                                             const float* __restrict__ rot,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse, int splits,
                                                             int hq, int hkv) {
  __shared__ float o1[D];
  const int r = blockIdx.x, c = threadIdx.x % RC;
  const int b = r / hq, hd = r - b * hq;
  const int s = b * hkv + hd / (hq / hkv);
  bool any = true;
  float l2 = 0.0f;
  for (int c0 = 0; c0 < D; c0 += RC) {
    float o;
    any = merge_splits<RG, RC>(part_ml + (uint64_t)r * splits * 2,
                               part_acc + (uint64_t)r * splits * D, splits, c0, &o, &l2);
    // `any` is uniform over the block: every thread takes the same path
    if (!any) break;
    if (threadIdx.x < RC) o1[c0 + c] = o;
    __syncthreads();  // the next slice rewrites the group states
  }
  static_assert(RG * RC >= D, "one thread per output channel");
  if (!any) {
    if (threadIdx.x < D) out[(uint64_t)r * D + threadIdx.x] = 0;
    if (lse && threadIdx.x == 0) lse[r] = -INFINITY;
    return;
  }
  if (threadIdx.x >= D) return;
  const int ch = threadIdx.x;
  const float* RV = rot + ((uint64_t)s * 2 + 1) * D * D + (uint64_t)ch * D;
  float v = 0.0f;
  for (int k = 0; k < D; ++k) v = __builtin_fmaf(RV[k], o1[k], v);
  out[(uint64_t)r * D + ch] = (uint16_t)f2bf(v);
  if (lse && ch == 0) lse[r] = l2 * 0.69314718055994530942f;
}

// Rotated queries for a rotated cache: q'[k] = fma chain over i of
// q[i] R_K[i][k] in fp32, stored as its bf16 rounding hi and the bf16
// rounding of the remainder lo.  grid (batch * hq), 128 threads: thread k.
__global__ __launch_bounds__(128) void k_rotate_q(const uint16_t* __restrict__ q,
                                                  const float* __restrict__ rot,
                                                  uint16_t* __restrict__ qhi,
                                                  uint16_t* __restrict__ qlo, int hq, int hkv) {
  const int r = blockIdx.x, k = threadIdx.x;
  const int b = r / hq, hd = r - b * hq;
  const int s = b * hkv + hd / (hq / hkv);
  const float* RK = rot + (uint64_t)s * 2 * D * D;
  const uint16_t* qr = q + (uint64_t)r * D;
  float acc = 0.0f;
  for (int i = 0; i < D; ++i) acc = __builtin_fmaf(bf2f(qr[i]), RK[i * D + k], acc);
  const uint32_t hi = f2bf(acc);
  qhi[(uint64_t)r * D + k] = (uint16_t)hi;
  qlo[(uint64_t)r * D + k] = (uint16_t)f2bf(acc - bf2f(hi));
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
  a.sl2 = p.scale * KVC_LOG2E;
  const dim3 grid((a.items + WAVES - 1) / WAVES);
  if (p.rot) {
    hipLaunchKernelGGL(k_rotate_q, dim3(p.batch * p.hq), dim3(128), 0, st, p.q, p.rot, p.qhi,
                       p.qlo, p.hq, p.hkv);
    if (p.G <= 4)
      hipLaunchKernelGGL((k_decode_split<1, true>), grid, dim3(64 * WAVES), 0, st, a);
    else if (p.G <= 8)
      hipLaunchKernelGGL((k_decode_split<2, true>), grid, dim3(64 * WAVES), 0, st, a);
    else
      hipLaunchKernelGGL((k_decode_split<4, true>), grid, dim3(64 * WAVES), 0, st, a);
    if (p.splits > 32)
      hipLaunchKernelGGL((k_decode_reduce_rot<32, 32>), dim3(p.batch * p.hq), dim3(1024), 0, st,
                         p.part_ml, p.part_acc, p.rot, p.out, p.lse, p.splits, p.hq, p.hkv);
    else if (p.splits > 8)
      hipLaunchKernelGGL((k_decode_reduce_rot<8, 128>), dim3(p.batch * p.hq), dim3(1024), 0, st,
                         p.part_ml, p.part_acc, p.rot, p.out, p.lse, p.splits, p.hq, p.hkv);
    else
      hipLaunchKernelGGL((k_decode_reduce_rot<1, 128>), dim3(p.batch * p.hq), dim3(128), 0, st,
                         p.part_ml, p.part_acc, p.rot, p.out, p.lse, p.splits, p.hq, p.hkv);
    return hipGetLastError();
  }
  if (p.G <= 4)
    hipLaunchKernelGGL((k_decode_split<1, false>), grid, dim3(64 * WAVES), 0, st, a);
  else if (p.G <= 8)
    hipLaunchKernelGGL((k_decode_split<2, false>), grid, dim3(64 * WAVES), 0, st, a);
  else
    hipLaunchKernelGGL((k_decode_split<4, false>), grid, dim3(64 * WAVES), 0, st, a);
  if (p.splits > 32)
    hipLaunchKernelGGL((k_decode_reduce<32, 32>), dim3(p.batch * p.hq, D / 32), dim3(1024), 0, st,
                       p.part_ml, p.part_acc, p.out, p.lse, p.splits);
  else if (p.splits > 8)
    hipLaunchKernelGGL((k_decode_reduce<8, 128>), dim3(p.batch * p.hq, 1), dim3(1024), 0, st,
                       p.part_ml, p.part_acc, p.out, p.lse, p.splits);
  else
    hipLaunchKernelGGL((k_decode_reduce<1, 128>), dim3(p.batch * p.hq, 1), dim3(128), 0, st,
                       p.part_ml, p.part_acc, p.out, p.lse, p.splits);
  return hipGetLastError();
}

}  // namespace kvc
