/*
 * kvc_oracle.c -- plain, slow CPU oracle for segment-wise two-dimensional
 * KV-cache compression and for decode attention over the compressed cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check
 * and the benchmark's CPU-baseline leg may load this library.  It shares no
 * code, header, table or constant with the HIP library; the two are compared
 * byte for byte (selection, indices, packed layout) and within a tolerance
 * (attention output).
 *
 * Sources (pages, with the passage each step follows):
 *  [M] "MosaicKV: Serving Long-Context LLM with Dynamic Two-D KV Cache
 *      Compression" (arXiv 2607.00760), review page: abstract (per-vector
 *      important elements, strategies chosen per KV segment); Fig. 5 caption
 *      (segments, strategy generation); Fig. 6 caption, Stage-1 (top-r
 *      elements of each KV vector), packed KV format, PackedAttention.
 *  [K] "KARA: Efficient Reasoning LLM Serving via Sliding-Window KV Cache
 *      Compression" (arXiv 2607.01237), review page: "What carries the
 *      argument" (keys of a recent window scored by attention accumulated
 *      from all window queries; Token2Chunk), referee summary (Eqs. 4-5
 *      bidirectional scoring, Eqs. 6-8 Token2Chunk), free-parameter ledger
 *      (retention r, window |W|, budget alpha, max length gamma), Fig. 3
 *      caption (bidirectional weights over all query/key pairs).
 *
 * The pages print no equations, so every numerical step below is the reading
 * stated beside it.  Selection-path arithmetic is IEEE fp32, round to nearest
 * even, no contraction except explicit fmaf, in exactly the order written;
 * attention is fp64.
 *
 * Parity pins (tests/test_oracle_pins.py) tie each function to closed forms,
 * brute force or textbook routines.  Token2Chunk's exact rule is not printed
 * on the pages: its properties are pinned, its parity with the paper is
 * unpinned.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <omp.h>

#define ORC_D 128           /* head dimension handled by the oracle */

/* ------------------------------------------------------------------ */
/* fp32 helpers                                                         */
/* ------------------------------------------------------------------ */
static float bf2f(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* log2(e) rounded to fp32, and the Taylor coefficients ln2^k / k!, k=0..7,
 * each rounded to fp32 (computed here in long double; a pin checks them
 * against the exactly rounded rationals). */
static float LOG2E_F;
static float EXPC[8];
static int g_init = 0;
static void orc_init(void) {
  if (g_init) return;
  const long double ln2 = 0.693147180559945309417232121458176568L;
  long double c = 1.0L;
  for (int k = 0; k < 8; ++k) {
    EXPC[k] = (float)c;
    c = c * ln2 / (long double)(k + 1);
  }
  LOG2E_F = (float)1.442695040888963407359924681001892137L;
  g_init = 1;
}

/* 2^y for y <= 0 by the Taylor series of e^(f ln2) (degree 7, Horner with
 * fmaf) after splitting y = n + f with n = rint(y), |f| <= 1/2; returns +0
 * below -125 so that no result is subnormal. */
static float orc_exp2(float y) {
  if (!(y >= -125.0f)) return 0.0f;
  float n = rintf(y);
  float f = y - n;
  float p = EXPC[7];
  for (int k = 6; k >= 0; --k) p = fmaf(p, f, EXPC[k]);
  return ldexpf(p, (int)n);
}

/* Pairwise sum over n entries, n a power of two: tree(a) = tree(first half)
 * + tree(second half). */
static float tree_pow2(const float* a, int n) {
  if (n == 1) return a[0];
  return tree_pow2(a, n / 2) + tree_pow2(a + n / 2, n / 2);
}
static int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}
/* Pairwise sum of n entries zero-padded to the next power of two. */
static float tree_any(const float* a, int n) {
  int np = next_pow2(n < 1 ? 1 : n);
  float* buf = (float*)calloc((size_t)np, sizeof(float));
  memcpy(buf, a, (size_t)n * sizeof(float));
  float r = tree_pow2(buf, np);
  free(buf);
  return r;
}

/* q . k as one fmaf chain over the channels in ascending order. */
static float dot_chain(const float* q, const uint16_t* k) {
  float acc = 0.0f;
  for (int ch = 0; ch < ORC_D; ++ch) acc = fmaf(q[ch], bf2f(k[ch]), acc);
  return acc;
}

/* ------------------------------------------------------------------ */
/* Public: element-wise exp2 and coefficient access (pins)             */
/* ------------------------------------------------------------------ */
void orc_exp2_f32(const float* y, float* out, long n) {
  orc_init();
  for (long i = 0; i < n; ++i) out[i] = orc_exp2(y[i]);
}
void orc_exp2_coeffs(float* c8, float* log2e) {
  orc_init();
  for (int k = 0; k < 8; ++k) c8[k] = EXPC[k];
  *log2e = LOG2E_F;
}

/* ------------------------------------------------------------------ */
/* Window scoring: accumulated attention of a window of queries        */
/*  [K] "What carries the argument": keys are scored by the attention   */
/*  all window queries give them; [K] Fig. 3: every query/key pair (no  */
/*  causal mask).  Reading: softmax of each query over the whole domain */
/*  of n_ctx keys, normalised globally; a token's score is the sum over */
/*  the G q-heads of its group and the W window queries.               */
/* ------------------------------------------------------------------ */
/* Qw: [nq][128] bf16, query index qi = g*W + w.  K: [n_ctx][128].
 * Outputs m[nq], invZ[nq]: for each query, m = the largest of its n_ctx
 * logits and Z = the pairwise sum (zero-padded to a power of two) over all
 * n_ctx tokens of exp(l - m); invZ = 1/Z. */
void orc_normalisers(int n_ctx, int nq, const uint16_t* K, const uint16_t* Qw,
                     float scale, float* m_out, float* invZ_out, int n_threads) {
  orc_init();
#pragma omp parallel for schedule(dynamic) num_threads(n_threads)
  for (int qi = 0; qi < nq; ++qi) {
    float q[ORC_D];
    for (int ch = 0; ch < ORC_D; ++ch) q[ch] = bf2f(Qw[(size_t)qi * ORC_D + ch]);
    float* l = (float*)malloc(sizeof(float) * (size_t)n_ctx);
    float m = -INFINITY;
    for (int t = 0; t < n_ctx; ++t) {
      l[t] = dot_chain(q, K + (size_t)t * ORC_D) * scale;
      if (l[t] > m) m = l[t];
    }
    for (int t = 0; t < n_ctx; ++t) l[t] = orc_exp2((l[t] - m) * LOG2E_F);
    const float Z = tree_any(l, n_ctx);
    m_out[qi] = m;
    invZ_out[qi] = 1.0f / Z;
    free(l);
  }
}

/* Scores of tokens [t0, t0+nt) of the domain: s = sum over qi ascending of
 * exp(l - m_qi) * invZ_qi, accumulated one term at a time. */
void orc_token_scores(int t0, int nt, int nq, const uint16_t* K, const uint16_t* Qw,
                      float scale, const float* m, const float* invZ, float* s_out,
                      int n_threads) {
  orc_init();
  float* qf = (float*)malloc(sizeof(float) * (size_t)nq * ORC_D);
  for (size_t i = 0; i < (size_t)nq * ORC_D; ++i) qf[i] = bf2f(Qw[i]);
#pragma omp parallel for schedule(static) num_threads(n_threads)
  for (int i = 0; i < nt; ++i) {
    const uint16_t* k = K + (size_t)(t0 + i) * ORC_D;
    float s = 0.0f;
    for (int qi = 0; qi < nq; ++qi) {
      float l = dot_chain(qf + (size_t)qi * ORC_D, k) * scale;
      float e = orc_exp2((l - m[qi]) * LOG2E_F);
      s = s + e * invZ[qi];
    }
    s_out[i] = s;
  }
  free(qf);
}

/* ------------------------------------------------------------------ */
/* Stage-1 per-vector channel selection ([M] Fig. 6 caption: the top-r  */
/* important elements of each K or V vector).  Reading: importance is  */
/* the magnitude of the stored bf16 value; order by magnitude (desc),   */
/* ties by lower channel; keep the first c.                             */
/* ------------------------------------------------------------------ */
typedef struct {
  uint16_t key;
  uint16_t ch;
} chkey;
static int cmp_chkey(const void* a, const void* b) {
  const chkey* x = (const chkey*)a;
  const chkey* y = (const chkey*)b;
  if (x->key != y->key) return x->key > y->key ? -1 : 1;
  return (int)x->ch - (int)y->ch;
}
/* mask: 16 bytes, channel ch -> byte ch/8, bit ch%8.  rho = share of the
 * vector's energy kept: pairwise sum of kept x^2 over pairwise sum of all
 * x^2 (1 when the vector is zero). */
void orc_channel_topc(const uint16_t* row, int c, uint8_t* mask, float* rho) {
  chkey ks[ORC_D];
  for (int ch = 0; ch < ORC_D; ++ch) {
    ks[ch].key = row[ch] & 0x7FFF;
    ks[ch].ch = (uint16_t)ch;
  }
  qsort(ks, ORC_D, sizeof(chkey), cmp_chkey);
  memset(mask, 0, 16);
  for (int i = 0; i < c && i < ORC_D; ++i) mask[ks[i].ch >> 3] |= (uint8_t)(1u << (ks[i].ch & 7));
  float kept[ORC_D], all[ORC_D];
  for (int ch = 0; ch < ORC_D; ++ch) {
    float x = bf2f(row[ch]);
    all[ch] = x * x;
    kept[ch] = ((mask[ch >> 3] >> (ch & 7)) & 1) ? all[ch] : 0.0f;
  }
  float Ec = tree_pow2(kept, ORC_D);
  float Ea = tree_pow2(all, ORC_D);
  *rho = (Ea == 0.0f) ? 1.0f : Ec / Ea;
}

/* ------------------------------------------------------------------ */
/* Token selection inside a segment                                     */
/* ------------------------------------------------------------------ */
typedef struct {
  float s;
  int idx;
} tokkey;
static int cmp_tokkey(const void* a, const void* b) {
  const tokkey* x = (const tokkey*)a;
  const tokkey* y = (const tokkey*)b;
  if (x->s != y->s) return x->s > y->s ? -1 : 1;
  return x->idx - y->idx;
}
/* Order of the segment's tokens by (score desc, index asc). */
static void token_order(const float* s, int S, int* order) {
  tokkey* t = (tokkey*)malloc(sizeof(tokkey) * (size_t)S);
  for (int i = 0; i < S; ++i) {
    t[i].s = s[i];
    t[i].idx = i;
  }
  qsort(t, (size_t)S, sizeof(tokkey), cmp_tokkey);
  for (int i = 0; i < S; ++i) order[i] = t[i].idx;
  free(t);
}
/* keep[i] = 1 for the T best tokens. */
void orc_top_t(const float* s, int S, int T, uint8_t* keep) {
  int* order = (int*)malloc(sizeof(int) * (size_t)S);
  token_order(s, S, order);
  memset(keep, 0, (size_t)S);
  for (int i = 0; i < T && i < S; ++i) keep[order[i]] = 1;
  free(order);
}

/* Token2Chunk ([K] "What carries the argument": consecutive high-score
 * tokens are endpoints of candidate chunks, the best kept under a length
 * cap and a budget; ledger: budget alpha, max chunk length gamma).
 * Reading: alpha tokens of the retention T are reserved for chunk interiors.
 *  1. A = the T - alpha best tokens, in ascending position a_1 < ... < a_m.
 *  2. Each neighbouring pair (a_k, a_k+1) with a gap (>= 1 token between)
 *     and span a_k+1 - a_k + 1 <= gamma is a candidate, valued
 *     s[a_k] + s[a_k+1] (fp32).
 *  3. Candidates are visited by (value desc, gap asc, k asc); one is accepted
 *     when its gap still fits the remaining budget (first fit), adding its
 *     interior tokens.
 *  4. Unused budget is filled with the best tokens not yet kept, so exactly
 *     T tokens are kept. */
void orc_token2chunk(const float* s, int S, int T, int alpha, int gamma, uint8_t* keep) {
  int* order = (int*)malloc(sizeof(int) * (size_t)S);
  token_order(s, S, order);
  memset(keep, 0, (size_t)S);
  int m = T - alpha;
  for (int i = 0; i < m; ++i) keep[order[i]] = 1;
  int* a = (int*)malloc(sizeof(int) * (size_t)(m > 0 ? m : 1));
  int na = 0;
  for (int i = 0; i < S; ++i)
    if (keep[i]) a[na++] = i;
  /* candidates */
  int nc = 0;
  int* ck = (int*)malloc(sizeof(int) * (size_t)(na > 0 ? na : 1));
  uint8_t* done = (uint8_t*)calloc((size_t)(na > 0 ? na : 1), 1);
  for (int k = 0; k + 1 < na; ++k) {
    int gap = a[k + 1] - a[k] - 1;
    int span = a[k + 1] - a[k] + 1;
    if (gap >= 1 && span <= gamma) ck[nc++] = k;
  }
  int used = 0;
  for (int it = 0; it < nc; ++it) {
    /* best remaining candidate by (value desc, gap asc, k asc) */
    int best = -1;
    float bv = 0.0f;
    int bg = 0;
    for (int j = 0; j < nc; ++j) {
      if (done[j]) continue;
      int k = ck[j];
      float v = s[a[k]] + s[a[k + 1]];
      int g = a[k + 1] - a[k] - 1;
      if (best < 0 || v > bv || (v == bv && (g < bg || (g == bg && k < ck[best])))) {
        best = j;
        bv = v;
        bg = g;
      }
    }
    done[best] = 1;
    if (used + bg <= alpha) {
      int k = ck[best];
      for (int t = a[k] + 1; t < a[k + 1]; ++t) keep[t] = 1;
      used += bg;
    }
  }
  /* fill to exactly T */
  int have = 0;
  for (int i = 0; i < S; ++i) have += keep[i];
  for (int i = 0; i < S && have < T; ++i) {
    if (!keep[order[i]]) {
      keep[order[i]] = 1;
      ++have;
    }
  }
  free(done);
  free(ck);
  free(a);
  free(order);
}

/* ------------------------------------------------------------------ */
/* Packed segment layout ([M] Fig. 6 caption: packed KV format, bf16   */
/* values + per-vector channel bitmask + token index list).  Parts,     */
/* each starting 16-byte aligned:                                       */
/*   K masks [T] x 16 B (only if c < 128), K values [T][c] bf16,        */
/*   V masks (only if c < 128), V values, token indices [T] u16 (only   */
/*   if T < S) zero-padded to 16 B.                                     */
/* K rows are token-major: token t's 16-byte mask (bit ch of byte ch/8, */
/* LSB first), and its kept values in channel order.                    */
/* V with c < 128 is grouped in blocks of 8 kept tokens (block b =      */
/* tokens 8b .. 8b+nb-1, nb = min(8, T - 8b)), each block transposed:   */
/* its mask bits fill bytes [128 b, 128 b + 16 nb) of the V mask part,  */
/* bit nb (2 l + h) + t (LSB first) set iff token 8b+t keeps channel    */
/* 64 h + l (l = 0..63, h = 0, 1); its values fill bytes                */
/* [16 c b, 16 c b + 2 c nb) of the V value part, the kept elements in  */
/* (l, h, t) order.  The page fixes the content (mask + kept values),   */
/* not the byte order; every part keeps the size above.  Dense V        */
/* (c = 128) is token-major.                                            */
/* ------------------------------------------------------------------ */
#define ORC_VBLK 8 /* tokens per transposed V block */
long orc_seg_bytes(int T, int c, int S) {
  if (T <= 0) return 0;
  long mk = (c < ORC_D) ? 16L * T : 0;
  long vals = 2L * T * c;
  long idx = (T < S) ? ((2L * T + 15) / 16) * 16 : 0;
  return 2 * mk + 2 * vals + idx;
}

/* V part of a masked segment in transposed 8-token blocks (layout above).
 * X: the segment's S rows [S][128] bf16; keep: S flags, T of them set;
 * out: 16 T mask bytes then 2 T c value bytes. */
static void orc_pack_v_blocks(const uint16_t* X, const uint8_t* keep, int S, int T, int c,
                              uint8_t* out) {
  int* tok = (int*)malloc(sizeof(int) * (size_t)T);
  uint8_t* mk = (uint8_t*)malloc((size_t)16 * T);
  int j = 0;
  for (int t = 0; t < S; ++t)
    if (keep[t]) tok[j++] = t;
  for (j = 0; j < T; ++j) {
    float r;
    orc_channel_topc(X + (size_t)tok[j] * ORC_D, c, mk + 16 * j, &r);
  }
  uint8_t* vm = out;
  uint8_t* vv = out + (size_t)16 * T;
  memset(vm, 0, (size_t)16 * T);
  for (int b = 0; ORC_VBLK * b < T; ++b) {
    const int nb = T - ORC_VBLK * b < ORC_VBLK ? T - ORC_VBLK * b : ORC_VBLK;
    uint8_t* bm = vm + (size_t)16 * ORC_VBLK * b;
    uint8_t* bv = vv + (size_t)2 * c * ORC_VBLK * b;
    int r = 0;
    for (int l = 0; l < 64; ++l)
      for (int h = 0; h < 2; ++h)
        for (int t = 0; t < nb; ++t) {
          const int jt = ORC_VBLK * b + t, ch = 64 * h + l;
          if (!((mk[16 * jt + (ch >> 3)] >> (ch & 7)) & 1)) continue;
          const int bit = nb * (2 * l + h) + t;
          bm[bit >> 3] |= (uint8_t)(1u << (bit & 7));
          memcpy(bv + 2 * r, &X[(size_t)tok[jt] * ORC_D + ch], 2);
          ++r;
        }
  }
  free(mk);
  free(tok);
}

/* Dense V rows [T][128] (bf16 bits, 0 where dropped) of a segment's V part:
 * vmask = the V mask part (masked segments), vval = the V value part. */
static void orc_v_dense(const uint8_t* vmask, const uint8_t* vval, int T, int c, uint16_t* out) {
  memset(out, 0, sizeof(uint16_t) * (size_t)T * ORC_D);
  if (c >= ORC_D) {
    memcpy(out, vval, sizeof(uint16_t) * (size_t)T * ORC_D);
    return;
  }
  for (int b = 0; ORC_VBLK * b < T; ++b) {
    const int nb = T - ORC_VBLK * b < ORC_VBLK ? T - ORC_VBLK * b : ORC_VBLK;
    const uint8_t* bm = vmask + (size_t)16 * ORC_VBLK * b;
    const uint8_t* bv = vval + (size_t)2 * c * ORC_VBLK * b;
    int r = 0;
    for (int l = 0; l < 64; ++l)
      for (int h = 0; h < 2; ++h)
        for (int t = 0; t < nb; ++t) {
          const int bit = nb * (2 * l + h) + t;
          if (!((bm[bit >> 3] >> (bit & 7)) & 1)) continue;
          memcpy(&out[(size_t)(ORC_VBLK * b + t) * ORC_D + 64 * h + l], bv + 2 * r, 2);
          ++r;
        }
  }
}

/* Descriptor, 16 bytes, same field order as the library's. */
typedef struct {
  uint64_t offset;
  uint16_t n_tok;
  uint16_t n_ch;
  uint8_t strategy;
  uint8_t flags;
  uint16_t seg_tokens;
} orc_desc;

typedef struct {
  int n_ctx;        /* tokens in the scoring domain */
  int region_begin; /* first token compressed */
  int region_len;   /* tokens compressed, a multiple of S */
  int S;            /* segment tokens */
  int G;            /* q heads per kv head */
  int W;            /* window queries per q head */
  int n_strat;
  const int* strat_T;
  const int* strat_c;
  long budget_bytes; /* per segment */
  int t2c_alpha;     /* 0: Token2Chunk off */
  int t2c_gamma;
  float scale;
  int budget_scope;  /* 0: each segment <= budget_bytes; 1: the stream's
                        segments together <= nseg * budget_bytes */
  int rotate;        /* 1: rotate the region's K and V vectors (SVD) before
                        channel selection and packing */
  int rot_span;      /* tokens per rotation span (0: the whole region) */
} orc_params;

/* ------------------------------------------------------------------ */
/* SVD rotation before the per-vector channel selection ([M] Fig. 6      */
/* caption, Stage-1: the SVD rotation matrix R of the K and of the V     */
/* matrix, respectively, is computed and the vectors are rotated before  */
/* the top-r elements of each are kept; Fig. 4: after the rotation the   */
/* important elements of the cache sit in a few channels).  Reading:     */
/*  - the region is cut into spans of rot_span tokens (one span = the    */
/*    whole region when rot_span is 0); each span has its own R for K    */
/*    and for V, from that span's vectors;                               */
/*  - R = the right singular vectors of the span's [T x 128] matrix X,   */
/*    i.e. the eigenvectors of the Gram matrix X^T X, ordered by          */
/*    eigenvalue (largest first, ties to the lower index);               */
/*  - a Gram entry is the dot product of two columns of X, computed like */
/*    every other dot product here: one fmaf chain in ascending token    */
/*    order;                                                             */
/*  - the eigenvectors come from cyclic Jacobi in fp32 with the          */
/*    round-robin (tournament) pair ordering of parallel Jacobi methods: */
/*    the 64 rotations of a round touch disjoint index pairs, so they are */
/*    all computed from the matrix as it stands and then applied as one  */
/*    similarity transform (rows, then columns), every operation fixed;  */
/*  - a vector x is stored as y = R^T x rounded to bf16; decode attends  */
/*    with R_K^T q in the span's basis and returns the sum over spans of */
/*    R_V times the span's share of the rotated output.                  */
/* ------------------------------------------------------------------ */
#define ORC_JACOBI_SWEEPS 10

static uint16_t f2bf_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* C[i][j] = sum over the T tokens of x_t[i] * x_t[j] as one fma chain in
 * ascending token order (a dot product of columns i and j of X). */
void orc_gram(const uint16_t* X, int T, float* C, int n_threads) {
#pragma omp parallel for schedule(dynamic) num_threads(n_threads)
  for (int i = 0; i < ORC_D; ++i) {
    for (int j = 0; j < ORC_D; ++j) {
      float acc = 0.0f;
      for (int t = 0; t < T; ++t)
        acc = fmaf(bf2f(X[(size_t)t * ORC_D + i]), bf2f(X[(size_t)t * ORC_D + j]), acc);
      C[i * ORC_D + j] = acc;
    }
  }
}

/* Pair k of round r of the round-robin ordering of 128 indices: index 127
 * meets r, and r + k meets r - k (mod 127) for k = 1..63; p < q. */
static void jacobi_pair(int r, int k, int* p, int* q) {
  int a, b;
  if (k == 0) {
    a = r;
    b = 127;
  } else {
    a = (r + k) % 127;
    b = (r - k + 127) % 127;
  }
  *p = a < b ? a : b;
  *q = a < b ? b : a;
}

/* Jacobi rotation that zeroes A[p][q]: tau = (A[q][q] - A[p][p]) / (2 A[p][q]),
 * t = sign(tau) / (|tau| + sqrt(tau^2 + 1)), c = 1 / sqrt(t^2 + 1), s = t c. */
static void jacobi_cs(float app, float aqq, float apq, float* c, float* s) {
  if (apq == 0.0f) {
    *c = 1.0f;
    *s = 0.0f;
    return;
  }
  const float tau = (aqq - app) / (2.0f * apq);
  const float t = (tau >= 0.0f ? 1.0f : -1.0f) / (fabsf(tau) + sqrtf(fmaf(tau, tau, 1.0f)));
  const float cc = 1.0f / sqrtf(fmaf(t, t, 1.0f));
  *c = cc;
  *s = t * cc;
}

/* Eigenvectors of the symmetric C: ORC_JACOBI_SWEEPS sweeps of 127 rounds;
 * in a round the 64 rotations are computed from A as it stands, then
 * applied to the rows of A, then to its columns, then to the columns of
 * the accumulated eigenvectors V (every element pair (a, b) of index p, q
 * becomes (fma(c, a, -(s b)), fma(s, a, c b))).  R[i][k] = V[i][order[k]]
 * with order sorting the diagonal of A (largest first, ties to the lower
 * index); evals[k] = that diagonal entry. */
void orc_jacobi(const float* C, float* R, float* evals) {
  float* A = (float*)malloc(sizeof(float) * ORC_D * ORC_D);
  float* V = (float*)malloc(sizeof(float) * ORC_D * ORC_D);
  memcpy(A, C, sizeof(float) * ORC_D * ORC_D);
  for (int i = 0; i < ORC_D * ORC_D; ++i) V[i] = 0.0f;
  for (int i = 0; i < ORC_D; ++i) V[i * ORC_D + i] = 1.0f;
  int P[64], Q[64];
  float cs[64], sn[64];
  for (int sweep = 0; sweep < ORC_JACOBI_SWEEPS; ++sweep) {
    for (int r = 0; r < 127; ++r) {
      for (int k = 0; k < 64; ++k) {
        jacobi_pair(r, k, &P[k], &Q[k]);
        jacobi_cs(A[P[k] * ORC_D + P[k]], A[Q[k] * ORC_D + Q[k]], A[P[k] * ORC_D + Q[k]], &cs[k],
                  &sn[k]);
      }
      for (int k = 0; k < 64; ++k) /* rows */
        for (int j = 0; j < ORC_D; ++j) {
          const float a = A[P[k] * ORC_D + j], b = A[Q[k] * ORC_D + j];
          A[P[k] * ORC_D + j] = fmaf(cs[k], a, -(sn[k] * b));
          A[Q[k] * ORC_D + j] = fmaf(sn[k], a, cs[k] * b);
        }
      for (int k = 0; k < 64; ++k) /* columns */
        for (int i = 0; i < ORC_D; ++i) {
          const float a = A[i * ORC_D + P[k]], b = A[i * ORC_D + Q[k]];
          A[i * ORC_D + P[k]] = fmaf(cs[k], a, -(sn[k] * b));
          A[i * ORC_D + Q[k]] = fmaf(sn[k], a, cs[k] * b);
        }
      for (int k = 0; k < 64; ++k) /* eigenvectors */
        for (int i = 0; i < ORC_D; ++i) {
          const float a = V[i * ORC_D + P[k]], b = V[i * ORC_D + Q[k]];
          V[i * ORC_D + P[k]] = fmaf(cs[k], a, -(sn[k] * b));
          V[i * ORC_D + Q[k]] = fmaf(sn[k], a, cs[k] * b);
        }
    }
  }
  int order[ORC_D];
  for (int k = 0; k < ORC_D; ++k) order[k] = k;
  for (int a = 1; a < ORC_D; ++a) { /* insertion sort: diagonal desc, index asc */
    const int o = order[a];
    int b = a - 1;
    while (b >= 0 && A[order[b] * ORC_D + order[b]] < A[o * ORC_D + o]) {
      order[b + 1] = order[b];
      --b;
    }
    order[b + 1] = o;
  }
  for (int k = 0; k < ORC_D; ++k) {
    evals[k] = A[order[k] * ORC_D + order[k]];
    for (int i = 0; i < ORC_D; ++i) R[i * ORC_D + k] = V[i * ORC_D + order[k]];
  }
  free(A);
  free(V);
}

/* y = R^T x rounded to bf16: y[k] = bf16(fma chain over i ascending of
 * x[i] R[i][k]). */
void orc_rotate(const uint16_t* X, long T, const float* R, uint16_t* Y) {
#pragma omp parallel for schedule(static)
  for (long t = 0; t < T; ++t)
    for (int k = 0; k < ORC_D; ++k) {
      float acc = 0.0f;
      for (int i = 0; i < ORC_D; ++i) acc = fmaf(bf2f(X[t * ORC_D + i]), R[i * ORC_D + k], acc);
      Y[t * ORC_D + k] = f2bf_rne(acc);
    }
}

/* ------------------------------------------------------------------ */
/* Per-stream byte budget ([M] abstract: compression strategies chosen   */
/* per KV segment under a memory target; Fig. 5 caption: strategy        */
/* generation).  Reading: a multiple-choice knapsack over the stream's   */
/* segments, maximise the sum of objectives J[sg][i] with the total      */
/* packed bytes <= B, solved by Lagrangian relaxation: for a multiplier  */
/* lambda >= 0 every segment takes argmax_i fl(J - fl(lambda * bytes_i)) */
/* (ties to the lower index); lambda is the smallest fp32 value, found   */
/* by binary search over the bit patterns 0 .. 2^97, whose total fits B  */
/* (2^97 x bytes stays finite and exceeds any objective difference, so   */
/* there every segment takes its smallest strategy, ties to the lower    */
/* index; if even that does not fit, that assignment is returned).  A    */
/* Lagrangian solution is optimal among all assignments that use at most */
/* its own bytes.                                                         */
/* ------------------------------------------------------------------ */
static uint64_t lagrange_pick(const float* J, const long* bytes, int nseg, int ns, float lambda,
                              int* chosen) {
  uint64_t tot = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    int best = 0;
    float bv = J[(size_t)sg * ns] - lambda * (float)bytes[0];
    for (int i = 1; i < ns; ++i) {
      const float v = J[(size_t)sg * ns + i] - lambda * (float)bytes[i];
      if (v > bv) {
        bv = v;
        best = i;
      }
    }
    chosen[sg] = best;
    tot += (uint64_t)bytes[best];
  }
  return tot;
}

static float bits_f(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Returns the multiplier's bit pattern. */
uint32_t orc_stream_choose(const float* J, const long* bytes, int nseg, int ns, uint64_t B,
                           int* chosen) {
  if (lagrange_pick(J, bytes, nseg, ns, 0.0f, chosen) <= B) return 0u;
  const uint32_t top = 0x70000000u; /* 2^97 */
  if (lagrange_pick(J, bytes, nseg, ns, bits_f(top), chosen) > B) return top;
  uint32_t lo = 0u, hi = top; /* total(lo) > B, total(hi) <= B */
  while (hi - lo > 1u) {
    const uint32_t mid = lo + (hi - lo) / 2u;
    if (lagrange_pick(J, bytes, nseg, ns, bits_f(mid), chosen) <= B)
      hi = mid;
    else
      lo = mid;
  }
  lagrange_pick(J, bytes, nseg, ns, bits_f(hi), chosen);
  return hi;
}

/* Compress one stream (one batch entry, one kv head).
 * K, V: [n_ctx][128] bf16; Qw: [G][W][128] bf16; forced: [nseg] or NULL
 * (value < n_strat forces a feasible strategy).  packed receives the stream's
 * segments back to back from byte 0; desc offsets are base_offset + local.
 * Optional outputs: scores [region_len], objective [nseg][n_strat],
 * m/invZ [G*W].  Returns 0, or -3 when no strategy fits the budget. */
int orc_compress_stream(const orc_params* p, const uint16_t* K, const uint16_t* V,
                        const uint16_t* Qw, const uint8_t* forced, uint8_t* packed,
                        uint64_t base_offset, orc_desc* desc, uint64_t* used_bytes,
                        float* scores_out, float* objective_out, float* m_out,
                        float* invZ_out, float* rot_out, int n_threads) {
  orc_init();
  /* rotation: selection and packing read the rotated region vectors
   * (scoring keeps the original keys); KS/VS index them by token - rb */
  const uint16_t* KS = K;
  const uint16_t* VS = V;
  long rb = 0;
  uint16_t *KR = NULL, *VR = NULL;
  if (p->rotate) {
    const int span = p->rot_span ? p->rot_span : p->region_len;
    if (span <= 0 || p->region_len % span) return -1;
    float* C = (float*)malloc(sizeof(float) * ORC_D * ORC_D);
    float* R = (float*)malloc(sizeof(float) * ORC_D * ORC_D);
    float ev[ORC_D];
    KR = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)p->region_len * ORC_D);
    VR = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)p->region_len * ORC_D);
    for (int sp = 0; sp < p->region_len / span; ++sp) {
      for (int side = 0; side < 2; ++side) {
        const size_t t0 = (size_t)sp * span;
        const uint16_t* X = (side ? V : K) + ((size_t)p->region_begin + t0) * ORC_D;
        orc_gram(X, span, C, n_threads);
        orc_jacobi(C, R, ev);
        orc_rotate(X, span, R, (side ? VR : KR) + t0 * ORC_D);
        if (rot_out)
          memcpy(rot_out + ((size_t)sp * 2 + side) * ORC_D * ORC_D, R,
                 sizeof(float) * ORC_D * ORC_D);
      }
    }
    free(C);
    free(R);
    KS = KR;
    VS = VR;
    rb = p->region_begin;
  }
  const int S = p->S, nseg = p->region_len / p->S, nq = p->G * p->W, ns = p->n_strat;
  if (p->budget_scope && forced) return -1;
  long* bytes = (long*)malloc(sizeof(long) * (size_t)ns);
  int any_feasible = 0;
  for (int i = 0; i < ns; ++i) {
    bytes[i] = orc_seg_bytes(p->strat_T[i], p->strat_c[i], S);
    if (bytes[i] <= p->budget_bytes) any_feasible = 1;
  }
  if (!any_feasible) {
    free(bytes);
    return -3;
  }
  /* 1. token scores over the region */
  float* m = (float*)malloc(sizeof(float) * (size_t)nq);
  float* invZ = (float*)malloc(sizeof(float) * (size_t)nq);
  float* s = (float*)malloc(sizeof(float) * (size_t)p->region_len);
  orc_normalisers(p->n_ctx, nq, K, Qw, p->scale, m, invZ, n_threads);
  orc_token_scores(p->region_begin, p->region_len, nq, K, Qw, p->scale, m, invZ, s, n_threads);
  if (scores_out) memcpy(scores_out, s, sizeof(float) * (size_t)p->region_len);
  if (m_out) memcpy(m_out, m, sizeof(float) * (size_t)nq);
  if (invZ_out) memcpy(invZ_out, invZ, sizeof(float) * (size_t)nq);

  /* 2. per segment: selection, objective, choice */
  int* chosen = (int*)malloc(sizeof(int) * (size_t)nseg);
  uint8_t* flags = (uint8_t*)calloc((size_t)nseg, 1);
  float* Jall = (float*)malloc(sizeof(float) * (size_t)nseg * (size_t)ns);
#pragma omp parallel for schedule(dynamic) num_threads(n_threads)
  for (int sg = 0; sg < nseg; ++sg) {
    const int t0 = p->region_begin + sg * S;
    const float* ss = s + (size_t)sg * S;
    float J[64];
    uint8_t* keep = (uint8_t*)malloc((size_t)S);
    float* terms = (float*)malloc(sizeof(float) * (size_t)S);
    /* energy shares of every K and V vector of the segment, per channel
     * count c < 128 that the strategy table uses (c = 128 keeps all: 1) */
    int cs[64], ncs = 0;
    for (int i = 0; i < ns; ++i) {
      int c = p->strat_c[i], seen = 0;
      if (p->strat_T[i] == 0 || c >= ORC_D) continue;
      for (int u = 0; u < ncs; ++u) seen |= (cs[u] == c);
      if (!seen) cs[ncs++] = c;
    }
    float* rhoK = (float*)malloc(sizeof(float) * (size_t)S * (size_t)(ncs > 0 ? ncs : 1));
    float* rhoV = (float*)malloc(sizeof(float) * (size_t)S * (size_t)(ncs > 0 ? ncs : 1));
    for (int t = 0; t < S; ++t) {
      for (int u = 0; u < ncs; ++u) {
        uint8_t mk[16];
        orc_channel_topc(KS + (size_t)(t0 - rb + t) * ORC_D, cs[u], mk, &rhoK[t * ncs + u]);
        orc_channel_topc(VS + (size_t)(t0 - rb + t) * ORC_D, cs[u], mk, &rhoV[t * ncs + u]);
      }
    }
    for (int i = 0; i < ns; ++i) {
      const int T = p->strat_T[i], c = p->strat_c[i];
      if (T == 0) {
        J[i] = 0.0f;
        continue;
      }
      if (T >= S)
        memset(keep, 1, (size_t)S);
      else if (p->t2c_alpha > 0)
        orc_token2chunk(ss, S, T, p->t2c_alpha, p->t2c_gamma, keep);
      else
        orc_top_t(ss, S, T, keep);
      int u = 0;
      while (u < ncs && cs[u] != c) ++u;
      /* objective: attention mass kept, weighted by the mean share of the
       * K and V vector energy kept at c channels */
      for (int t = 0; t < S; ++t) {
        if (!keep[t]) {
          terms[t] = 0.0f;
          continue;
        }
        float rk = 1.0f, rv = 1.0f;
        if (c < ORC_D) {
          rk = rhoK[t * ncs + u];
          rv = rhoV[t * ncs + u];
        }
        terms[t] = ss[t] * (0.5f * (rk + rv));
      }
      J[i] = tree_pow2(terms, S);
    }
    free(rhoK);
    free(rhoV);
    int best = -1;
    if (forced && forced[sg] < ns && bytes[forced[sg]] <= p->budget_bytes) {
      best = forced[sg];
    } else {
      if (forced && forced[sg] != 0xFF) flags[sg] |= 0x80;
      for (int i = 0; i < ns; ++i) {
        if (bytes[i] > p->budget_bytes) continue;
        if (best < 0 || J[i] > J[best]) best = i;
      }
    }
    chosen[sg] = best;
    for (int i = 0; i < ns; ++i) Jall[(size_t)sg * ns + i] = J[i];
    if (objective_out)
      for (int i = 0; i < ns; ++i) objective_out[(size_t)sg * ns + i] = J[i];
    free(keep);
    free(terms);
  }

  if (p->budget_scope)
    orc_stream_choose(Jall, bytes, nseg, ns, (uint64_t)p->budget_bytes * (uint64_t)nseg, chosen);
  free(Jall);

  /* 3. offsets (exclusive scan) and 4. pack */
  uint64_t off = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    const int i = chosen[sg], T = p->strat_T[i], c = p->strat_c[i];
    const int t0 = p->region_begin + sg * S;
    const long nb = bytes[i];
    orc_desc d;
    memset(&d, 0, sizeof d);
    d.offset = base_offset + off;
    d.n_tok = (uint16_t)T;
    d.n_ch = (uint16_t)(T > 0 ? c : 0);
    d.strategy = (uint8_t)i;
    d.flags = (uint8_t)(flags[sg] | (T >= S ? 1 : 0) | (c >= ORC_D ? 2 : 0));
    d.seg_tokens = (uint16_t)S;
    desc[sg] = d;
    uint8_t* out = packed + off;
    memset(out, 0, (size_t)nb);
    if (T > 0) {
      uint8_t* keep = (uint8_t*)malloc((size_t)S);
      if (T >= S)
        memset(keep, 1, (size_t)S);
      else if (p->t2c_alpha > 0)
        orc_token2chunk(s + (size_t)sg * S, S, T, p->t2c_alpha, p->t2c_gamma, keep);
      else
        orc_top_t(s + (size_t)sg * S, S, T, keep);
      size_t pos = 0;
      for (int part = 0; part < 2; ++part) { /* 0: K, 1: V */
        const uint16_t* X = part == 0 ? KS : VS;
        if (part == 1 && c < ORC_D) {
          orc_pack_v_blocks(X + (size_t)(t0 - rb) * ORC_D, keep, S, T, c, out + pos);
          pos += (size_t)16 * T + (size_t)2 * T * c;
          continue;
        }
        if (c < ORC_D) {
          for (int t = 0; t < S; ++t) {
            if (!keep[t]) continue;
            float r;
            orc_channel_topc(X + (size_t)(t0 - rb + t) * ORC_D, c, out + pos, &r);
            pos += 16;
          }
        }
        for (int t = 0; t < S; ++t) {
          if (!keep[t]) continue;
          const uint16_t* row = X + (size_t)(t0 - rb + t) * ORC_D;
          uint8_t mk[16];
          float r;
          if (c < ORC_D)
            orc_channel_topc(row, c, mk, &r);
          else
            memset(mk, 0xFF, 16);
          for (int ch = 0; ch < ORC_D; ++ch) {
            if ((mk[ch >> 3] >> (ch & 7)) & 1) {
              memcpy(out + pos, &row[ch], 2);
              pos += 2;
            }
          }
        }
      }
      if (T < S) {
        for (int t = 0; t < S; ++t) {
          if (!keep[t]) continue;
          uint16_t u = (uint16_t)t;
          memcpy(out + pos, &u, 2);
          pos += 2;
        }
      }
      free(keep);
    }
    off += (uint64_t)nb;
  }
  *used_bytes = off;
  free(chosen);
  free(flags);
  free(m);
  free(invZ);
  free(s);
  free(bytes);
  free(KR);
  free(VR);
  return 0;
}

/* ------------------------------------------------------------------ */
/* Decode attention over a compressed stream ([M] Fig. 6/7 captions:    */
/* PackedAttention computes attention over the packed KV).  Exact       */
/* (fp64) softmax attention over every kept token; a dropped channel    */
/* contributes 0 to q.k and to the output.                              */
/* q: [G][128] bf16.  desc: n_desc descriptors whose offsets index      */
/* packed.  out: [G][128] fp64, lse: [G] (log of the softmax            */
/* denominator incl. the max; -inf and out = 0 if no token is kept).     */
/* ------------------------------------------------------------------ */
/* Tokens a descriptor's parts are sized for: n_tok, or seg_tokens for a
 * paged descriptor (flags bit2), whose first n_tok of seg_tokens rows are
 * filled so that tokens can be appended in place. */
static int layout_tokens(const orc_desc* d) { return (d->flags & 4) ? d->seg_tokens : d->n_tok; }
static int max_tok(const orc_desc* d, int n) {
  int m = 0;
  for (int i = 0; i < n; ++i) m = d[i].n_tok > m ? d[i].n_tok : m;
  return m;
}

static void decode_core(int G, const double* qd, const uint8_t* packed, const orc_desc* desc,
                        int n_desc, float scale, double* out, double* lse);

void orc_decode_stream(int G, const uint16_t* q, const uint8_t* packed, const orc_desc* desc,
                       int n_desc, float scale, double* out, double* lse) {
  double* qd = (double*)malloc(sizeof(double) * (size_t)G * ORC_D);
  for (int i = 0; i < G * ORC_D; ++i) qd[i] = (double)bf2f(q[i]);
  decode_core(G, qd, packed, desc, n_desc, scale, out, lse);
  free(qd);
}

/* Decode over a cache stored in the rotated bases (compressed with
 * rotation): rot holds [n_span][2][128][128] fp32 (R_K, R_V of each span),
 * descriptor i belongs to span i / desc_per_span.  Exact attention over the
 * stored vectors with the logits of token t taken against q' = R_K^T q of
 * t's span; out = sum over spans of R_V times the softmax-weighted sum of
 * that span's stored V vectors; all in fp64 from the fp32 matrices. */
void orc_decode_stream_rot(int G, const uint16_t* q, const uint8_t* packed, const orc_desc* desc,
                           int n_desc, float scale, const float* rot, int desc_per_span,
                           double* out, double* lse) {
  const int n_span = (n_desc + desc_per_span - 1) / desc_per_span;
  double* qd = (double*)calloc((size_t)n_span * G * ORC_D + 1, sizeof(double));
  for (int sp = 0; sp < n_span; ++sp) {
    const float* RK = rot + (size_t)sp * 2 * ORC_D * ORC_D;
    for (int g = 0; g < G; ++g)
      for (int k = 0; k < ORC_D; ++k) {
        double acc = 0.0;
        for (int i = 0; i < ORC_D; ++i)
          acc += (double)bf2f(q[g * ORC_D + i]) * (double)RK[i * ORC_D + k];
        qd[((size_t)sp * G + g) * ORC_D + k] = acc;
      }
  }
  /* logits of every kept token against its span's rotated query */
  long ntok = 0;
  for (int i = 0; i < n_desc; ++i) ntok += desc[i].n_tok;
  double* l = (double*)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1) * (size_t)G);
  long j = 0;
  for (int i = 0; i < n_desc; ++i) {
    const double* qs = qd + (size_t)(i / desc_per_span) * G * ORC_D;
    const int T = desc[i].n_tok, c = desc[i].n_ch, TL = layout_tokens(&desc[i]);
    const uint8_t* base = packed + desc[i].offset;
    const uint8_t* kval = base + (c < ORC_D ? 16 * TL : 0);
    for (int t = 0; t < T; ++t, ++j) {
      const uint8_t* mk = c < ORC_D ? base + 16 * t : NULL;
      const uint8_t* vals = kval + (size_t)2 * c * t;
      for (int g = 0; g < G; ++g) {
        double acc = 0.0;
        int r = 0;
        for (int ch = 0; ch < ORC_D; ++ch) {
          if (mk && !((mk[ch >> 3] >> (ch & 7)) & 1)) continue;
          uint16_t u;
          memcpy(&u, vals + 2 * r, 2);
          ++r;
          acc += qs[g * ORC_D + ch] * (double)bf2f(u);
        }
        l[(size_t)j * G + g] = acc * (double)scale;
      }
    }
  }
  double* o1 = (double*)calloc((size_t)G * ORC_D + 1, sizeof(double));
  uint16_t* vd = (uint16_t*)malloc(sizeof(uint16_t) * ORC_D * (size_t)(max_tok(desc, n_desc) + 1));
  double* mx = (double*)malloc(sizeof(double) * (size_t)G);
  double* den = (double*)malloc(sizeof(double) * (size_t)G);
  for (int g = 0; g < G; ++g) {
    for (int i = 0; i < ORC_D; ++i) out[g * ORC_D + i] = 0.0;
    mx[g] = -INFINITY;
    den[g] = 0.0;
    if (ntok == 0) {
      lse[g] = -INFINITY;
      continue;
    }
    for (long t = 0; t < ntok; ++t) mx[g] = l[t * G + g] > mx[g] ? l[t * G + g] : mx[g];
    for (long t = 0; t < ntok; ++t) den[g] += exp(l[t * G + g] - mx[g]);
    lse[g] = mx[g] + log(den[g]);
  }
  /* per span: the weighted sum of its stored V vectors, then R_V times it */
  j = 0;
  for (int sp = 0; ntok > 0 && sp < n_span; ++sp) {
    for (int k = 0; k < G * ORC_D; ++k) o1[k] = 0.0;
    const int i1 = (sp + 1) * desc_per_span < n_desc ? (sp + 1) * desc_per_span : n_desc;
    for (int i = sp * desc_per_span; i < i1; ++i) {
      const int T = desc[i].n_tok, c = desc[i].n_ch, TL = layout_tokens(&desc[i]);
      const uint8_t* base = packed + desc[i].offset;
      const size_t mb = c < ORC_D ? (size_t)16 * TL : 0;
      const uint8_t* vmask = base + mb + (size_t)2 * TL * c;
      orc_v_dense(vmask, vmask + mb, T, c, vd);
      for (int t = 0; t < T; ++t, ++j)
        for (int g = 0; g < G; ++g) {
          const double pw = exp(l[(size_t)j * G + g] - mx[g]) / den[g];
          for (int ch = 0; ch < ORC_D; ++ch)
            o1[g * ORC_D + ch] += pw * (double)bf2f(vd[(size_t)t * ORC_D + ch]);
        }
    }
    const float* RV = rot + ((size_t)sp * 2 + 1) * ORC_D * ORC_D;
    for (int g = 0; g < G; ++g)
      for (int i = 0; i < ORC_D; ++i) {
        double acc = 0.0;
        for (int k = 0; k < ORC_D; ++k) acc += (double)RV[i * ORC_D + k] * o1[g * ORC_D + k];
        out[g * ORC_D + i] += acc;
      }
  }
  free(den);
  free(mx);
  free(vd);
  free(o1);
  free(l);
  free(qd);
}

static void decode_core(int G, const double* qd, const uint8_t* packed, const orc_desc* desc,
                        int n_desc, float scale, double* out, double* lse) {
  long ntok = 0;
  for (int i = 0; i < n_desc; ++i) ntok += desc[i].n_tok;
  double* l = (double*)malloc(sizeof(double) * (size_t)(ntok > 0 ? ntok : 1) * (size_t)G);
  uint16_t* vd = (uint16_t*)malloc(sizeof(uint16_t) * ORC_D * (size_t)(max_tok(desc, n_desc) + 1));
  /* pass 1: logits */
  long j = 0;
  for (int i = 0; i < n_desc; ++i) {
    const int T = desc[i].n_tok, c = desc[i].n_ch, TL = layout_tokens(&desc[i]);
    const uint8_t* base = packed + desc[i].offset;
    const uint8_t* kmask = base;
    const uint8_t* kval = base + (c < ORC_D ? 16 * TL : 0);
    for (int t = 0; t < T; ++t, ++j) {
      const uint8_t* mk = c < ORC_D ? kmask + 16 * t : NULL;
      const uint8_t* vals = kval + (size_t)2 * c * t;
      for (int g = 0; g < G; ++g) {
        double acc = 0.0;
        int r = 0;
        for (int ch = 0; ch < ORC_D; ++ch) {
          int on = mk ? ((mk[ch >> 3] >> (ch & 7)) & 1) : 1;
          if (!on) continue;
          uint16_t kv;
          memcpy(&kv, vals + 2 * r, 2);
          ++r;
          acc += qd[g * ORC_D + ch] * (double)bf2f(kv);
        }
        l[j * G + g] = acc * (double)scale;
      }
    }
  }
  double* mx = (double*)malloc(sizeof(double) * (size_t)G);
  double* den = (double*)malloc(sizeof(double) * (size_t)G);
  for (int g = 0; g < G; ++g) {
    for (int ch = 0; ch < ORC_D; ++ch) out[g * ORC_D + ch] = 0.0;
    mx[g] = -INFINITY;
    den[g] = 0.0;
    if (ntok == 0) {
      lse[g] = -INFINITY;
      continue;
    }
    for (long t = 0; t < ntok; ++t)
      if (l[t * G + g] > mx[g]) mx[g] = l[t * G + g];
    for (long t = 0; t < ntok; ++t) den[g] += exp(l[t * G + g] - mx[g]);
    lse[g] = mx[g] + log(den[g]);
  }
  /* pass 2: weighted sum of the kept V elements, token by token (a dropped
   * element is a stored zero, which adds nothing) */
  long jj = 0;
  for (int i = 0; i < n_desc; ++i) {
    const int T = desc[i].n_tok, c = desc[i].n_ch, TL = layout_tokens(&desc[i]);
    const uint8_t* base = packed + desc[i].offset;
    const size_t kpart = (size_t)(c < ORC_D ? 16 * TL : 0) + (size_t)2 * TL * c;
    const uint8_t* vmask = base + kpart;
    orc_v_dense(vmask, vmask + (c < ORC_D ? 16 * TL : 0), T, c, vd);
    for (int t = 0; t < T; ++t, ++jj)
      for (int g = 0; g < G; ++g) {
        const double pr = exp(l[jj * G + g] - mx[g]) / den[g];
        for (int ch = 0; ch < ORC_D; ++ch)
          out[g * ORC_D + ch] += pr * (double)bf2f(vd[(size_t)t * ORC_D + ch]);
      }
  }
  free(den);
  free(mx);
  free(vd);
  free(l);
}

/* ------------------------------------------------------------------ */
/* Query-aware segment selection at decode time ([M] Fig. 6 caption:    */
/* stage 2 runs during decode before each attention layer; Sec. 5.3:    */
/* PackedAttention performs sequence compression in each attention      */
/* layer of the decode stage; Fig. 8: token selection rates 6.25 % and  */
/* 12.5 %; Quest, the query-aware page selection the page compares      */
/* against).  Reading: per segment, the per-channel maximum and minimum */
/* of its decoded keys (a dropped channel counts as 0); per q head an   */
/* upper bound of q.k over the segment, sum over channels of            */
/* max(q kmax, q kmin); a segment's score is the largest bound over     */
/* the group's heads; the k best segments by (score desc, index asc)    */
/* are kept, in index order.                                            */
/* ------------------------------------------------------------------ */

/* summary: [n_desc][2][128] bf16 bits: kmax, kmin of each descriptor's
 * kept K vectors (zeros for an empty descriptor).  Zeros are taken as +0,
 * so that the maximum and minimum do not depend on the token order. */
void orc_summarize_stream(const uint8_t* packed, const orc_desc* desc, int n_desc,
                          uint16_t* summary) {
  for (int i = 0; i < n_desc; ++i) {
    const int T = desc[i].n_tok, c = desc[i].n_ch, TL = layout_tokens(&desc[i]);
    uint16_t* smax = summary + (size_t)i * 2 * ORC_D;
    uint16_t* smin = smax + ORC_D;
    const uint8_t* base = packed + desc[i].offset;
    const uint8_t* kval = base + (c < ORC_D ? 16 * TL : 0);
    float mx[ORC_D], mn[ORC_D];
    for (int ch = 0; ch < ORC_D; ++ch) {
      mx[ch] = -INFINITY;
      mn[ch] = INFINITY;
    }
    for (int t = 0; t < T; ++t) {
      const uint8_t* mk = c < ORC_D ? base + 16 * t : NULL;
      const uint8_t* vals = kval + (size_t)2 * c * t;
      int r = 0;
      for (int ch = 0; ch < ORC_D; ++ch) {
        float x = 0.0f;
        int on = mk ? ((mk[ch >> 3] >> (ch & 7)) & 1) : 1;
        if (on) {
          uint16_t kv;
          memcpy(&kv, vals + 2 * r, 2);
          ++r;
          x = bf2f(kv) + 0.0f; /* -0 counts as +0, so the range has one bit pattern */
        }
        if (x > mx[ch]) mx[ch] = x;
        if (x < mn[ch]) mn[ch] = x;
      }
    }
    for (int ch = 0; ch < ORC_D; ++ch) {
      float a = T > 0 ? mx[ch] : 0.0f, b = T > 0 ? mn[ch] : 0.0f;
      uint32_t ua, ub;
      memcpy(&ua, &a, 4);
      memcpy(&ub, &b, 4);
      smax[ch] = (uint16_t)(ua >> 16); /* exact: every candidate is a bf16 value */
      smin[ch] = (uint16_t)(ub >> 16);
    }
  }
}

/* Score of one segment: max over the G heads of the pairwise-tree fp32
 * sum over channels 0..127 (the selection path's summation order) of
 * max(q kmax, q kmin); each product of two bf16 values is exact in fp32. */
static float segment_score(int G, const uint16_t* q, const uint16_t* sm) {
  float best = -INFINITY;
  float term[ORC_D];
  for (int g = 0; g < G; ++g) {
    for (int ch = 0; ch < ORC_D; ++ch) {
      const float qv = bf2f(q[g * ORC_D + ch]);
      const float a = qv * bf2f(sm[ch]), b = qv * bf2f(sm[ORC_D + ch]);
      term[ch] = (a > b ? a : b) + 0.0f; /* -0 counts as +0 (a q element may be -0) */
    }
    const float acc = tree_pow2(term, ORC_D);
    if (acc > best) best = acc;
  }
  return best;
}

typedef struct {
  float s;
  int i;
} seg_key;
static int cmp_segkey(const void* a, const void* b) {
  const seg_key* x = (const seg_key*)a;
  const seg_key* y = (const seg_key*)b;
  if (x->s != y->s) return x->s > y->s ? -1 : 1;
  return x->i - y->i;
}

/* q: [G][128] bf16; summary from orc_summarize_stream.  Writes the score of
 * every descriptor (-inf for an empty one) and the indices of the kept
 * descriptors in ascending order; returns their number, min(k, non-empty). */
int orc_select_stream(int G, const uint16_t* q, const uint16_t* summary, const orc_desc* desc,
                      int n_desc, int k, float* score, int* sel) {
  seg_key* keys = (seg_key*)malloc(sizeof(seg_key) * (size_t)(n_desc > 0 ? n_desc : 1));
  int m = 0;
  for (int i = 0; i < n_desc; ++i) {
    score[i] = desc[i].n_tok > 0 ? segment_score(G, q, summary + (size_t)i * 2 * ORC_D) : -INFINITY;
    if (desc[i].n_tok > 0) {
      keys[m].s = score[i];
      keys[m].i = i;
      ++m;
    }
  }
  qsort(keys, (size_t)m, sizeof(seg_key), cmp_segkey);
  const int n = k < m ? k : m;
  uint8_t* on = (uint8_t*)calloc((size_t)(n_desc > 0 ? n_desc : 1), 1);
  for (int j = 0; j < n; ++j) on[keys[j].i] = 1;
  int w = 0;
  for (int i = 0; i < n_desc; ++i)
    if (on[i]) sel[w++] = i;
  free(on);
  free(keys);
  return n;
}

int orc_max_threads(void) { return omp_get_max_threads(); }
