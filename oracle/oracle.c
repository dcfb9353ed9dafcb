/*
 * CPU reference checker for block-sparse attention (test infrastructure).
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg use
 * this file.  It shares no code with the GPU library: plain C, fp64
 * arithmetic, OpenMP across independent rows, no blocking or fusion.
 *
 * What each routine computes and where the pages define it:
 *
 *  oracle_build_csr   Block mask -> per-row ascending KV-block lists.  A row is
 *                     one (batch, query head, query block); an entry is kept
 *                     when mask != 0, or when the threshold T <= p
 *                     (ScalingAttention, section 5.2, Eq. 2: M_p = I(T <= p)),
 *                     or when it is the row's diagonal block (always kept).
 *                     The ascending order is the order in which the CRM
 *                     forward iterator of ScalingAttention (section 7.3,
 *                     Algorithm 2) walks the active KV blocks.  Log-weights
 *                     are copied bit for bit from the log-weight map.
 *  oracle_build_crm   Block mask -> CRM rows (ScalingAttention, section 7.2:
 *                     Compressed Row Mask): each row is an array of
 *                     ceil(nKB / 32) uint32 words, bit (v mod 32) of word
 *                     (v / 32) set when KV block v is kept (same keep rule
 *                     as oracle_build_csr); bits at v >= nKB stay clear.
 *  oracle_crm_walk    The CRM forward iterator (ScalingAttention, section 7.3,
 *                     Algorithm 2) run over every row: the state holds the
 *                     next word, the last word, the current word's remaining
 *                     bits and the index of its bit 0 (one word before the
 *                     row at the start); loading a word moves that index on
 *                     by 32, a cleared word loads the next one, each step
 *                     yields base + count-trailing-zeros and clears the
 *                     lowest bit.  Bits of the last word at v >= nKB are
 *                     not part of the row and are skipped.  Writes the
 *                     yielded indices as CSR.
 *  oracle_perm_from_labels
 *                     Gather permutation that makes every cluster contiguous
 *                     (InstaGen, section 4: tokens permuted into contiguous
 *                     blocks by cluster); ties keep the original order.
 *  oracle_schedule    Query-row order: KV-group-major over heads
 *                     (WaveAlign, section VI-B: sequential-head scheduling),
 *                     consecutive buckets of at most W rows each sorted by
 *                     descending nonzero-block count (WaveAlign, section IV-D,
 *                     NNZ-guided intra-wave alignment), then the launch-index
 *                     remap that gives each XCD a contiguous run.
 *                     An optional per-head row order (below) replaces the
 *                     query-block order inside each segment.  With a head
 *                     step of 2 only the first head of each pair of query
 *                     heads that share a KV head is scheduled (one launch
 *                     serves the pair's identical rows).
 *  oracle_schedule_pairs
 *                     The same sequence and buckets, with consecutive query
 *                     blocks of a head that list identical blocks served by
 *                     one launch entry (two rows, one staging of each K/V
 *                     tile; the library's reading of the K/V-reuse motive of
 *                     WaveAlign, section IV): greedy pairing along each head,
 *                     entries sorted by their tile count, the second row of
 *                     a pair leaving an empty entry at the bucket's end.
 *  oracle_spectral_order
 *                     WaveAlign stage 1 (section IV-C): rank-2 embedding of
 *                     each head's mask rows by matrix-free centred subspace
 *                     iteration (IV-C.2), rows ordered by polar angle (IV-C.1).
 *  oracle_attn_rows   Dense-masked softmax attention, InstaGen section 3.1
 *                     Eq. (1)-(3), with the per-block log-weight added to the
 *                     scaled logit (InstaGen Algorithm 1, Horvitz-Thompson
 *                     weights as log w).  Masked pairs are -inf.
 *  oracle_segment_offsets / oracle_segment_means
 *                     Centroids for InstaGen Algorithm 1 step 2: the tokens
 *                     of each label form one contiguous segment of the
 *                     label-sorted sequence, and a centroid is the mean of
 *                     its segment's rows (fixed-length segments give the mean
 *                     key of each 128-key tile).
 *  oracle_is_sample   Group-shared importance sampling over KV tiles
 *                     (InstaGen Algorithm 1 steps 2-13, section 3.2.1
 *                     Eq. 4): centroid scores, the exact set by decreasing
 *                     size x score, water-filled inclusion probabilities,
 *                     a systematic PPS sample, Horvitz-Thompson log-weights.
 *  oracle_attn_tok    Token-level attention over computational query sets
 *                     (INTRA, sections 3 and 4.8: a CQS is a group of query
 *                     tokens given by a query mapping, attending to the key
 *                     tokens given by a key mapping; outputs go back to the
 *                     query positions).  InstaGen Eq. (1)-(3) over the
 *                     CQS's key list, one term per list entry; entries
 *                     outside the sequence and, when causal, keys after the
 *                     query are left out.
 *  oracle_group_mass  MC-Sparse's exact token selection, second pass: the
 *                     attention probabilities of every query of a group
 *                     (softmax over all keys, the dense first pass's LSE)
 *                     summed per key over the group's queries.
 *  oracle_topk        The K keys of largest mass per row (MC-Sparse's top-K
 *                     on the aggregated mass), ties to the lower index,
 *                     listed in ascending order.
 *  oracle_count_pairs Number of allowed (query, key) token pairs; the FLOP
 *                     convention of 4*d per pair is the one behind INTRA's
 *                     GFLOPS column (INTRA, Table 1 and the overhead table).
 *
 * Every function is pinned by the CPU test suite against something other
 * than itself (library routines, brute force, closed forms, invariants).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG (-1)
#define OR_ERR_CAPACITY (-3)

static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* mask -> CSR                                                               */
/* ------------------------------------------------------------------------ */
static int kept(const uint8_t *mask, const float *T, float p, int64_t r, int64_t v,
                int64_t nQB, int64_t nKB, int force_diag) {
  int64_t i = r * nKB + v;
  int k;
  if (mask)
    k = mask[i] != 0;
  else
    k = T[i] <= p; /* NaN compares false */
  if (force_diag && v == r % nQB) k = 1;
  return k;
}

/* Fills row_ptr[R+1]; when col != NULL also col (and lw when lw != NULL).
 * Returns nnz, or a negative error. */
int64_t oracle_build_csr(const uint8_t *mask, const float *T, float p, const float *lw_map,
                         int64_t R, int64_t nQB, int64_t nKB, int force_diag, int32_t *row_ptr,
                         int32_t *col, float *lw, int64_t capacity) {
  if ((!mask && !T) || R < 0 || nQB <= 0 || nKB <= 0 || !row_ptr) return OR_ERR_ARG;
  int64_t n = 0;
  row_ptr[0] = 0;
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t v = 0; v < nKB; ++v) {
      if (!kept(mask, T, p, r, v, nQB, nKB, force_diag)) continue;
      if (col) {
        if (n >= capacity) return OR_ERR_CAPACITY;
        col[n] = (int32_t)v;
        if (lw) {
          if (lw_map)
            memcpy(&lw[n], &lw_map[r * nKB + v], sizeof(float));
          else
            lw[n] = 0.0f;
        }
      }
      ++n;
    }
    row_ptr[r + 1] = (int32_t)n;
  }
  return n;
}

/* ------------------------------------------------------------------------ */
/* mask -> CRM, CRM -> CSR by the forward iterator                           */
/* ------------------------------------------------------------------------ */
/* words[r * W + v / 32] bit v % 32, W = ceil(nKB / 32). */
int oracle_build_crm(const uint8_t *mask, const float *T, float p, int64_t R, int64_t nQB,
                     int64_t nKB, int force_diag, uint32_t *words) {
  if ((!mask && !T) || R < 0 || nQB <= 0 || nKB <= 0 || !words) return OR_ERR_ARG;
  int64_t W = (nKB + 31) / 32;
  for (int64_t r = 0; r < R; ++r) {
    uint32_t *row = words + r * W;
    for (int64_t w = 0; w < W; ++w) row[w] = 0u;
    for (int64_t v = 0; v < nKB; ++v)
      if (kept(mask, T, p, r, v, nQB, nKB, force_diag)) row[v / 32] |= (uint32_t)1 << (v % 32);
  }
  return OR_OK;
}

/* Iterator state over one row's words. */
typedef struct {
  const uint32_t *ptr, *end; /* next word to load, one past the last */
  uint32_t val;              /* bits of the current word not yet yielded */
  int64_t base;              /* KV-block index of bit 0 of the current word */
  uint32_t tail;             /* bits of the last word that name blocks below nKB */
} crm_iter;

static int trailing_zeros(uint32_t x) { /* x != 0 */
  int n = 0;
  while (!(x & 1u)) {
    x >>= 1;
    ++n;
  }
  return n;
}

/* Loads words until one with a set bit is current or the row is used up. */
static void crm_advance(crm_iter *s) {
  while (s->val == 0u && s->ptr < s->end) {
    s->val = *s->ptr++;
    if (s->ptr == s->end) s->val &= s->tail;
    s->base += 32;
  }
}

/* Fills row_ptr[R+1]; when col != NULL also col.  Returns nnz, or a negative
 * error. */
int64_t oracle_crm_walk(const uint32_t *words, int64_t R, int64_t nKB, int32_t *row_ptr, int32_t *col,
                        int64_t capacity) {
  if (!words || R < 0 || nKB <= 0 || !row_ptr) return OR_ERR_ARG;
  int64_t W = (nKB + 31) / 32, n = 0;
  row_ptr[0] = 0;
  for (int64_t r = 0; r < R; ++r) {
    crm_iter s = {words + r * W, words + (r + 1) * W, 0u, -32,
                  nKB % 32 ? ((uint32_t)1 << (nKB % 32)) - 1u : ~0u};
    crm_advance(&s);
    while (s.val != 0u) {
      if (col) {
        if (n >= capacity) return OR_ERR_CAPACITY;
        col[n] = (int32_t)(s.base + trailing_zeros(s.val));
      }
      ++n;
      s.val &= s.val - 1u;
      if (s.val == 0u) crm_advance(&s);
    }
    row_ptr[r + 1] = (int32_t)n;
  }
  return n;
}

/* ------------------------------------------------------------------------ */
/* labels -> permutation                                                     */
/* ------------------------------------------------------------------------ */
typedef struct {
  int64_t key;
  int32_t idx;
} key_idx;

static int cmp_key_idx(const void *a, const void *b) {
  const key_idx *x = (const key_idx *)a, *y = (const key_idx *)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

/* perm[bh][i] = original index of the token at permuted position i, sorted by
 * (label, original index).  Labels outside [0, n_clusters) sort after every
 * valid label. */
int oracle_perm_from_labels(const int32_t *labels, int64_t BH, int64_t N, int32_t n_clusters,
                            int32_t *perm) {
  if (!labels || !perm || BH < 0 || N < 0 || n_clusters <= 0) return OR_ERR_ARG;
  key_idx *buf = (key_idx *)malloc(sizeof(key_idx) * (size_t)(N > 0 ? N : 1));
  if (!buf) return OR_ERR_ARG;
  for (int64_t bh = 0; bh < BH; ++bh) {
    for (int64_t i = 0; i < N; ++i) {
      int32_t l = labels[bh * N + i];
      buf[i].key = (l >= 0 && l < n_clusters) ? l : n_clusters;
      buf[i].idx = (int32_t)i;
    }
    qsort(buf, (size_t)N, sizeof(key_idx), cmp_key_idx);
    for (int64_t i = 0; i < N; ++i) perm[bh * N + i] = buf[i].idx;
  }
  free(buf);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* row schedule                                                              */
/* ------------------------------------------------------------------------ */
/* Logical sequence: for each batch b and KV head g, the rows of the G = Hq/Hkv
 * query heads that share g, position u outer and head inner; position u is
 * query block u, or query block row_perm[head][u] when a per-head order is
 * given.  Buckets of
 * at most W consecutive entries within one (b, g) segment are sorted by
 * (nnz descending, sequence position ascending).  With n_xcd > 1 the list is
 * then dealt so that launch index i runs logical position start(i % n_xcd) +
 * i / n_xcd, where XCD x receives the x-th contiguous slice.
 *
 * W = 0 takes buckets of 2048 entries.  With W = 0 and the block lists (col)
 * given, each bucket keeps whichever of two orders lets consecutive rows
 * share more KV blocks (the rows an XCD runs one after another; WaveAlign,
 * section IV: the schedule exists for K/V reuse in L2): the sorted order
 * above, or the sequence order itself.  Shared blocks are estimated with a
 * 256-bit signature per row (bit v mod 256 for every listed block v, v read
 * as unsigned): the cost of an order is the sum over its rows of the bits
 * set in a row's signature and not in the previous row's (the first row:
 * all of its bits); the sequence order is kept when its cost is smaller,
 * and then sorted by (nnz descending, position ascending) within each window
 * of 64 consecutive entries of the bucket (WaveAlign's intra-wave alignment
 * over two XCD-waves of rows). */
static int sig_fresh(const uint64_t *a, const uint64_t *prev) {
  int c = 0;
  for (int w = 0; w < 4; ++w) {
    uint64_t x = a[w] & ~(prev ? prev[w] : 0ull);
    while (x) {
      x &= x - 1;
      ++c;
    }
  }
  return c;
}

int oracle_schedule(const int32_t *row_ptr, const int32_t *col, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t nQB, int64_t W, int64_t n_xcd, const int32_t *row_perm, int64_t head_step,
                    int32_t *order) {
  if (!row_ptr || !order || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || nQB <= 0 || W < 0)
    return OR_ERR_ARG;
  const int adaptive = W == 0 && col != NULL;
  if (W == 0) W = 2048;
  if (head_step < 1 || (Hq / Hkv) % head_step) return OR_ERR_ARG;
  /* rows scheduled: heads g*G + j with j a multiple of head_step */
  int64_t G = Hq / Hkv, Gs = G / head_step, R = B * Hkv * Gs * nQB, seg = Gs * nQB;
  int32_t *logical = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
  key_idx *buf = (key_idx *)malloc(sizeof(key_idx) * (size_t)W);
  if (!logical || !buf) return OR_ERR_ARG;
  int64_t pos = 0;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t g = 0; g < Hkv; ++g)
      for (int64_t u = 0; u < nQB; ++u)
        for (int64_t j = 0; j < Gs; ++j) {
          int64_t h = b * Hq + g * G + j * head_step;
          int64_t uu = row_perm ? row_perm[h * nQB + u] : u;
          logical[pos++] = (int32_t)(h * nQB + uu);
        }
  uint64_t *sig = adaptive ? (uint64_t *)calloc((size_t)W * 4, sizeof(uint64_t)) : NULL;
  if (adaptive && !sig) return OR_ERR_ARG;
  for (int64_t s0 = 0; s0 < R; s0 += seg) {
    for (int64_t b0 = s0; b0 < s0 + seg; b0 += W) {
      int64_t n = (b0 + W <= s0 + seg) ? W : s0 + seg - b0;
      for (int64_t i = 0; i < n; ++i) {
        int32_t r = logical[b0 + i];
        buf[i].key = -(int64_t)(row_ptr[r + 1] - row_ptr[r]);
        buf[i].idx = (int32_t)i;
      }
      qsort(buf, (size_t)n, sizeof(key_idx), cmp_key_idx);
      if (adaptive) {
        for (int64_t i = 0; i < n; ++i) {
          uint64_t *si = sig + 4 * i;
          si[0] = si[1] = si[2] = si[3] = 0;
          int32_t r = logical[b0 + i];
          for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
            uint32_t bit = (uint32_t)col[e] % 256u;
            si[bit / 64] |= 1ull << (bit % 64);
          }
        }
        int64_t cost_sorted = 0, cost_seq = 0;
        for (int64_t i = 0; i < n; ++i) {
          cost_seq += sig_fresh(sig + 4 * i, i ? sig + 4 * (i - 1) : NULL);
          cost_sorted += sig_fresh(sig + 4 * buf[i].idx, i ? sig + 4 * buf[i - 1].idx : NULL);
        }
        if (cost_seq < cost_sorted) {   /* the sequence order, sorted within windows of 64 */
          for (int64_t w0 = 0; w0 < n; w0 += 64) {
            int64_t m = w0 + 64 <= n ? 64 : n - w0;
            for (int64_t i = 0; i < m; ++i) {
              int32_t r = logical[b0 + w0 + i];
              buf[i].key = -(int64_t)(row_ptr[r + 1] - row_ptr[r]);
              buf[i].idx = (int32_t)i;
            }
            qsort(buf, (size_t)m, sizeof(key_idx), cmp_key_idx);
            int32_t t[64];
            for (int64_t i = 0; i < m; ++i) t[i] = logical[b0 + w0 + buf[i].idx];
            memcpy(&logical[b0 + w0], t, sizeof(int32_t) * (size_t)m);
          }
          continue;
        }
      }
      int32_t tmp[4096];
      int32_t *t = n <= 4096 ? tmp : (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
      for (int64_t i = 0; i < n; ++i) t[i] = logical[b0 + buf[i].idx];
      memcpy(&logical[b0], t, sizeof(int32_t) * (size_t)n);
      if (t != tmp) free(t);
    }
  }
  if (n_xcd <= 1) {
    memcpy(order, logical, sizeof(int32_t) * (size_t)R);
  } else {
    for (int64_t i = 0; i < R; ++i) {
      int64_t x = i % n_xcd, k = i / n_xcd, start = 0;
      for (int64_t y = 0; y < x; ++y) start += (R - 1 - y) / n_xcd + 1; /* launches on XCD y */
      order[i] = logical[start + k];
    }
  }
  free(sig);
  free(buf);
  free(logical);
  return OR_OK;
}

/* Launch tables with paired rows.  The sequence, segments, buckets (W; 0
 * takes 2048 and, with col, the adaptive order) and the XCD deal are those of
 * oracle_schedule with head step 1.  Inside a bucket, positions i and i + G
 * hold consecutive query blocks of one head (G = Hq / Hkv query heads per
 * segment, head inner).  Walking the bucket's positions in ascending order,
 * a position that is not already the second row of a pair is paired with
 * position i + G when that position lies in the bucket and the two rows list
 * the same blocks in the same order with the same log-weight bits (lw
 * optional); otherwise it is a single entry.  An entry's cost is its tile
 * count: nnz for a single row, 2 nnz for a pair.  Entries are ordered by
 * (cost descending, position ascending); with the adaptive order, the
 * signature cost of section "row schedule" above is taken over entries (the
 * first row's signature) in that order and in position order, and when the
 * position order is cheaper the entries keep it, sorted by (cost descending,
 * position ascending) within each window of 64 positions.  The second rows
 * of pairs follow as empty entries (-1, -1) in position order.  order[i]
 * receives an entry's first row, order2[i] its second row or -1. */
int oracle_schedule_pairs(const int32_t *row_ptr, const int32_t *col, const float *lw, int64_t B, int64_t Hq,
                          int64_t Hkv, int64_t nQB, int64_t W, int64_t n_xcd, const int32_t *row_perm,
                          int32_t *order, int32_t *order2) {
  if (!row_ptr || !col || !order || !order2 || B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || nQB <= 0 || W < 0)
    return OR_ERR_ARG;
  const int adaptive = W == 0;
  if (W == 0) W = 2048;
  const int64_t G = Hq / Hkv, R = B * Hq * nQB, seg = G * nQB;
  int32_t *l1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
  int32_t *l2 = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
  int32_t *logical = (int32_t *)malloc(sizeof(int32_t) * (size_t)R);
  int8_t *kind = (int8_t *)malloc((size_t)W); /* 0 single, 1 first of a pair, 2 second */
  key_idx *buf = (key_idx *)malloc(sizeof(key_idx) * (size_t)W);
  int32_t *units = (int32_t *)malloc(sizeof(int32_t) * (size_t)W);
  uint64_t *sig = (uint64_t *)calloc((size_t)W * 4, sizeof(uint64_t));
  if (!l1 || !l2 || !logical || !kind || !buf || !units || !sig) return OR_ERR_ARG;
  int64_t pos = 0;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t g = 0; g < Hkv; ++g)
      for (int64_t u = 0; u < nQB; ++u)
        for (int64_t j = 0; j < G; ++j) {
          int64_t h = b * Hq + g * G + j;
          int64_t uu = row_perm ? row_perm[h * nQB + u] : u;
          logical[pos++] = (uu >= 0 && uu < nQB) ? (int32_t)(h * nQB + uu) : -1;
        }
  for (int64_t s0 = 0; s0 < R; s0 += seg) {
    for (int64_t b0 = s0; b0 < s0 + seg; b0 += W) {
      int64_t n = (b0 + W <= s0 + seg) ? W : s0 + seg - b0;
      const int32_t *rw = logical + b0;
      /* greedy pairing */
      memset(kind, 0, (size_t)n);
      for (int64_t i = 0; i < n; ++i) {
        if (kind[i] == 2 || i + G >= n) continue;
        int32_t a = rw[i], c = rw[i + G];
        if (a < 0 || c < 0) continue;
        int32_t la = row_ptr[a + 1] - row_ptr[a], lc = row_ptr[c + 1] - row_ptr[c];
        int same = la == lc;
        for (int32_t e = 0; same && e < la; ++e) {
          if (col[row_ptr[a] + e] != col[row_ptr[c] + e]) same = 0;
          if (lw) {
            uint32_t x, y;
            memcpy(&x, &lw[row_ptr[a] + e], 4);
            memcpy(&y, &lw[row_ptr[c] + e], 4);
            if (x != y) same = 0;
          }
        }
        if (same) {
          kind[i] = 1;
          kind[i + G] = 2;
        }
      }
      /* entries in position order, with their costs */
      int64_t m = 0;
      for (int64_t i = 0; i < n; ++i) {
        if (kind[i] == 2) continue;
        int32_t r = rw[i];
        int64_t nnz = r >= 0 ? row_ptr[r + 1] - row_ptr[r] : 0;
        buf[m].key = -(kind[i] == 1 ? 2 * nnz : nnz);
        buf[m].idx = (int32_t)i;
        units[m] = (int32_t)i;
        ++m;
      }
      qsort(buf, (size_t)m, sizeof(key_idx), cmp_key_idx);
      if (adaptive) {
        for (int64_t i = 0; i < n; ++i) {
          uint64_t *si = sig + 4 * i;
          si[0] = si[1] = si[2] = si[3] = 0;
          int32_t r = rw[i];
          if (r < 0) continue;
          for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
            uint32_t bit = (uint32_t)col[e] % 256u;
            si[bit / 64] |= 1ull << (bit % 64);
          }
        }
        int64_t cost_sorted = 0, cost_seq = 0;
        for (int64_t t = 0; t < m; ++t) {
          cost_seq += sig_fresh(sig + 4 * units[t], t ? sig + 4 * units[t - 1] : NULL);
          cost_sorted += sig_fresh(sig + 4 * buf[t].idx, t ? sig + 4 * buf[t - 1].idx : NULL);
        }
        if (cost_seq < cost_sorted) { /* position order, sorted within windows of 64 positions */
          for (int64_t t = 0; t < m; ++t) {
            int32_t i = units[t];
            int32_t r = rw[i];
            int64_t nnz = r >= 0 ? row_ptr[r + 1] - row_ptr[r] : 0;
            buf[t].key = (int64_t)(i / 64) * ((int64_t)1 << 40) - (kind[i] == 1 ? 2 * nnz : nnz);
            buf[t].idx = i;
          }
          qsort(buf, (size_t)m, sizeof(key_idx), cmp_key_idx);
        }
      }
      int64_t t = 0;
      for (; t < m; ++t) {
        int32_t i = buf[t].idx;
        l1[b0 + t] = rw[i];
        l2[b0 + t] = kind[i] == 1 ? rw[i + G] : -1;
      }
      for (int64_t i = 0; i < n; ++i)
        if (kind[i] == 2) {
          l1[b0 + t] = -1;
          l2[b0 + t] = -1;
          ++t;
        }
    }
  }
  for (int64_t i = 0; i < R; ++i) {
    int64_t src = i;
    if (n_xcd > 1) {
      int64_t x = i % n_xcd, k = i / n_xcd, start = 0;
      for (int64_t y = 0; y < x; ++y) start += (R - 1 - y) / n_xcd + 1; /* launches on XCD y */
      src = start + k;
    }
    order[i] = l1[src];
    order2[i] = l2[src];
  }
  free(sig);
  free(units);
  free(buf);
  free(kind);
  free(logical);
  free(l2);
  free(l1);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* WaveAlign stage 1: polar spectral row order                               */
/* ------------------------------------------------------------------------ */
/* For every head bh (rows r = bh*nQB + u, u = 0..nQB-1) its mask M is the
 * nQB x nKB 0/1 matrix of the listed blocks (entries outside [0, nKB) are
 * ignored).  The centred mask C = M - 1 mu^T, mu[v] = (1/nQB) sum_u M[u][v],
 * keeps pairwise row distances and sends the constant (workload) direction
 * to a zero singular value (WaveAlign, section IV-C.2).  Its top-2 left
 * singular subspace is found by subspace iteration X <- orth(C C^T X),
 * applied without forming C: C^T X = M^T X - mu (1^T X) and
 * C Z = M Z - 1 (mu^T Z).  The start is
 *   X0[i] = ( ((37 i + 11) mod 101) / 101 - 1/2, ((53 i + 29) mod 97) / 97 - 1/2 )
 * and orth is Gram-Schmidt on the two columns (a zero column stays zero).
 * Row i is then placed by the polar angle atan2(X[i][1], X[i][0]) of its
 * coordinates (section IV-C.1), ties by i.
 * Out: perm[bh*nQB + p] = query block at position p; angle[bh*nQB + i] (or
 * NULL). */
static int cmp_angle_idx(const void *a, const void *b) {
  const double *x = (const double *)a, *y = (const double *)b;
  if (x[0] < y[0]) return -1;
  if (x[0] > y[0]) return 1;
  return (x[1] > y[1]) - (x[1] < y[1]);
}

static void orth2(double *x1, double *x2, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += x1[i] * x1[i];
  double nrm = sqrt(s);
  for (int64_t i = 0; i < n; ++i) x1[i] = nrm > 0.0 ? x1[i] / nrm : 0.0;
  double d = 0.0;
  for (int64_t i = 0; i < n; ++i) d += x1[i] * x2[i];
  for (int64_t i = 0; i < n; ++i) x2[i] -= d * x1[i];
  s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += x2[i] * x2[i];
  nrm = sqrt(s);
  for (int64_t i = 0; i < n; ++i) x2[i] = nrm > 0.0 ? x2[i] / nrm : 0.0;
}

int oracle_spectral_order(const int32_t *row_ptr, const int32_t *col, int64_t BH, int64_t nQB, int64_t nKB,
                          int64_t iters, int32_t *perm, double *angle) {
  if (!row_ptr || !col || !perm || BH <= 0 || nQB <= 0 || nKB <= 0 || iters < 1) return OR_ERR_ARG;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < BH; ++bh) {
    double *x1 = malloc(sizeof(double) * nQB), *x2 = malloc(sizeof(double) * nQB);
    double *y1 = malloc(sizeof(double) * nQB), *y2 = malloc(sizeof(double) * nQB);
    double *z1 = malloc(sizeof(double) * nKB), *z2 = malloc(sizeof(double) * nKB);
    double *mu = calloc((size_t)nKB, sizeof(double));
    double *key = malloc(sizeof(double) * 2 * nQB);
    if (!x1 || !x2 || !y1 || !y2 || !z1 || !z2 || !mu || !key) {
#pragma omp atomic write
      bad = 1;
    } else {
      const int32_t *rp = row_ptr + bh * nQB;
      for (int64_t u = 0; u < nQB; ++u)
        for (int32_t e = rp[u]; e < rp[u + 1]; ++e)
          if (col[e] >= 0 && col[e] < nKB) mu[col[e]] += 1.0;
      for (int64_t v = 0; v < nKB; ++v) mu[v] /= (double)nQB;
      for (int64_t i = 0; i < nQB; ++i) {
        x1[i] = (double)((37 * i + 11) % 101) / 101.0 - 0.5;
        x2[i] = (double)((53 * i + 29) % 97) / 97.0 - 0.5;
      }
      for (int64_t it = 0; it < iters; ++it) {
        /* Z = C^T X */
        double s1 = 0.0, s2 = 0.0;
        for (int64_t i = 0; i < nQB; ++i) {
          s1 += x1[i];
          s2 += x2[i];
        }
        for (int64_t v = 0; v < nKB; ++v) z1[v] = z2[v] = 0.0;
        for (int64_t u = 0; u < nQB; ++u)
          for (int32_t e = rp[u]; e < rp[u + 1]; ++e)
            if (col[e] >= 0 && col[e] < nKB) {
              z1[col[e]] += x1[u];
              z2[col[e]] += x2[u];
            }
        for (int64_t v = 0; v < nKB; ++v) {
          z1[v] -= mu[v] * s1;
          z2[v] -= mu[v] * s2;
        }
        /* Y = C Z */
        double t1 = 0.0, t2 = 0.0;
        for (int64_t v = 0; v < nKB; ++v) {
          t1 += mu[v] * z1[v];
          t2 += mu[v] * z2[v];
        }
        for (int64_t u = 0; u < nQB; ++u) {
          double a1 = 0.0, a2 = 0.0;
          for (int32_t e = rp[u]; e < rp[u + 1]; ++e)
            if (col[e] >= 0 && col[e] < nKB) {
              a1 += z1[col[e]];
              a2 += z2[col[e]];
            }
          y1[u] = a1 - t1;
          y2[u] = a2 - t2;
        }
        orth2(y1, y2, nQB);
        memcpy(x1, y1, sizeof(double) * nQB);
        memcpy(x2, y2, sizeof(double) * nQB);
      }
      for (int64_t i = 0; i < nQB; ++i) {
        key[2 * i] = atan2(x2[i], x1[i]);
        key[2 * i + 1] = (double)i;
        if (angle) angle[bh * nQB + i] = key[2 * i];
      }
      qsort(key, (size_t)nQB, 2 * sizeof(double), cmp_angle_idx);
      for (int64_t p = 0; p < nQB; ++p) perm[bh * nQB + p] = (int32_t)key[2 * p + 1];
    }
    free(x1); free(x2); free(y1); free(y2); free(z1); free(z2); free(mu); free(key);
  }
  return bad ? OR_ERR_ARG : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* WaveAlign adaptive skip of stage 1                                        */
/* ------------------------------------------------------------------------ */
/* WaveAlign, section IV-E (Runtime Coordination) and section VI-F with
 * Figure 13: the reordering is bypassed when its estimated latency reduction
 * does not exceed its overhead; reordering was skipped at low retained
 * densities (1.7 %, 6.7 %) and enabled from 14.5 %.  The pages give the
 * estimate in words only; this is the reading, step by step:
 *   nnz   = listed entries over all BH heads (each entry is one tile the
 *           attention kernel processes, whatever block it names);
 *   nmax  = the largest per-head nnz (heads are reordered in parallel);
 *   fresh = sum over rows of the entries whose block the row before it in
 *           the same head does not list (the first row of a head: all), so
 *           f = fresh / nnz is the share of K/V block visits that the
 *           current order does not pair with the previous row;
 *   density = nnz / (BH nQB nKB);
 *   t_attn  = nnz * tile_ms * (block/128)^2 * (d/128) / n_cus, the attention
 *             time at the measured cost of one block pair on one compute unit;
 *   gain    = gamma * f * t_attn;
 *   cost    = (iters / 10) * (row_ms * nQB + nnz_ms * nmax);
 *   footprint = 2 * N * d * 2 bytes of K and V per KV head.
 * Stage 1 runs when footprint > l2_bytes (otherwise every block stays in the
 * L2 whatever the order), density >= density_min, gain > cost, and the
 * stage-1 kernel supports the shape (nQB, nKB <= 1024, nKB * ceil(nQB/32)
 * and nQB * ceil(nKB/32) <= 12288).  prm = {gamma, tile_ms, row_ms, nnz_ms,
 * density_min, l2_bytes}.  stats (out, 7 doubles): f, density, t_attn,
 * gain, cost, footprint, and the decision as 0/1. */
int oracle_stage1_decide(const int32_t *row_ptr, const int32_t *col, int64_t BH, int64_t nQB, int64_t nKB,
                         int64_t N, int64_t d, int64_t block, int64_t iters, int64_t n_cus, const double *prm,
                         int32_t *run, double *stats) {
  if (!row_ptr || !col || !prm || !run || BH <= 0 || nQB <= 0 || nKB <= 0 || N <= 0 || d <= 0 ||
      block <= 0 || iters < 1 || n_cus <= 0)
    return OR_ERR_ARG;
  int64_t nnz = 0, nmax = 0, fresh = 0;
  for (int64_t h = 0; h < BH; ++h) {
    int64_t nh = 0;
    for (int64_t u = 0; u < nQB; ++u) {
      const int64_t r = h * nQB + u;
      for (int64_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
        const int32_t v = col[e];
        ++nh;
        int in_prev = 0;
        if (u > 0)
          for (int64_t e2 = row_ptr[r - 1]; e2 < row_ptr[r]; ++e2)
            if (col[e2] == v) in_prev = 1;
        if (!in_prev) ++fresh;
      }
    }
    nnz += nh;
    if (nh > nmax) nmax = nh;
  }
  const double gamma = prm[0], tile_ms = prm[1], row_ms = prm[2], nnz_ms = prm[3], density_min = prm[4],
               l2_bytes = prm[5];
  const double f = nnz > 0 ? (double)fresh / (double)nnz : 0.0;
  const double density = (double)nnz / ((double)BH * (double)nQB * (double)nKB);
  const double bs = (double)block / 128.0;
  const double t_attn = (double)nnz * tile_ms * bs * bs * ((double)d / 128.0) / (double)n_cus;
  const double gain = gamma * f * t_attn;
  const double cost = ((double)iters / 10.0) * (row_ms * (double)nQB + nnz_ms * (double)nmax);
  const double footprint = 4.0 * (double)N * (double)d;
  const int64_t w1 = (nQB + 31) / 32, w2 = (nKB + 31) / 32;
  const int supported = nQB <= 1024 && nKB <= 1024 && nKB * w1 <= 12288 && nQB * w2 <= 12288;
  const int go = supported && footprint > l2_bytes && density >= density_min && gain > cost;
  *run = go;
  if (stats) {
    stats[0] = f;
    stats[1] = density;
    stats[2] = t_attn;
    stats[3] = gain;
    stats[4] = cost;
    stats[5] = footprint;
    stats[6] = (double)go;
  }
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* attention                                                                 */
/* ------------------------------------------------------------------------ */
/* rows[i] = (b * Hq + h) * N + t with t an original (unpermuted) token index.
 * Strides are in elements for (batch, head, token); the head dimension is
 * contiguous.  perm_q is [B*Hq][N], perm_k is [B*Hkv][N] (gather form: the
 * original index at each permuted position) or NULL for the identity.
 * out[i*d .. i*d+d-1] and lse[i] receive O and ln(sum exp) of that row; a row
 * with no allowed key gets O = 0 and LSE = -inf. */
int oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const int64_t *q_str, const int64_t *k_str, const int64_t *v_str, int64_t B,
                     int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t block,
                     const int32_t *row_ptr, const int32_t *col, const float *lw,
                     const int32_t *perm_q, const int32_t *perm_k, int causal, double scale,
                     int64_t n_rows, const int64_t *rows, double *out, double *lse) {
  if (!q || !k || !v || !row_ptr || !col || !rows || !out || B <= 0 || Hq <= 0 || Hkv <= 0 ||
      Hq % Hkv || N <= 0 || d <= 0 || block <= 0)
    return OR_ERR_ARG;
  int64_t G = Hq / Hkv, nQB = (N + block - 1) / block, nKB = nQB;
  /* permuted position of every original token */
  int32_t *pos_q = NULL, *pos_k = NULL;
  if (perm_q) {
    pos_q = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B * Hq * N));
    for (int64_t bh = 0; bh < B * Hq; ++bh)
      for (int64_t i = 0; i < N; ++i) pos_q[bh * N + perm_q[bh * N + i]] = (int32_t)i;
  }
  if (perm_k) {
    pos_k = (int32_t *)malloc(sizeof(int32_t) * (size_t)(B * Hkv * N));
    for (int64_t bh = 0; bh < B * Hkv; ++bh)
      for (int64_t i = 0; i < N; ++i) pos_k[bh * N + perm_k[bh * N + i]] = (int32_t)i;
  }
  int bad = 0;
#pragma omp parallel
  {
    double *x = (double *)malloc(sizeof(double) * (size_t)N);
    char *allowed = (char *)malloc((size_t)N);
    char *present = (char *)malloc((size_t)nKB);
    double *bias = (double *)malloc(sizeof(double) * (size_t)nKB);
    double *qv = (double *)malloc(sizeof(double) * (size_t)d);
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t i = 0; i < n_rows; ++i) {
      int64_t flat = rows[i];
      int64_t bh = flat / N, t = flat % N;
      if (bh < 0 || bh >= B * Hq) {
        bad = 1;
        continue;
      }
      int64_t b = bh / Hq, h = bh % Hq, g = h / G, bg = b * Hkv + g;
      int64_t pq = pos_q ? pos_q[bh * N + t] : t;
      int64_t u = pq / block;
      int64_t r = bh * nQB + u;
      memset(present, 0, (size_t)nKB);
      for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
        present[col[e]] = 1;
        bias[col[e]] = lw ? (double)lw[e] : 0.0;
      }
      const uint16_t *qrow = q + b * q_str[0] + h * q_str[1] + t * q_str[2];
      for (int64_t c = 0; c < d; ++c) qv[c] = bf16_to_double(qrow[c]);
      double m = -INFINITY;
      for (int64_t s = 0; s < N; ++s) {
        int64_t ps = pos_k ? pos_k[bg * N + s] : s;
        int64_t vb = ps / block;
        allowed[s] = present[vb] && !(causal && s > t);
        if (!allowed[s]) continue;
        const uint16_t *krow = k + b * k_str[0] + g * k_str[1] + s * k_str[2];
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qv[c] * bf16_to_double(krow[c]);
        x[s] = scale * dot + bias[vb];
        if (x[s] > m) m = x[s];
      }
      for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
      double Z = 0.0;
      if (m != -INFINITY) {
        for (int64_t s = 0; s < N; ++s) {
          if (!allowed[s]) continue;
          double w = exp(x[s] - m);
          Z += w;
          const uint16_t *vrow = v + b * v_str[0] + g * v_str[1] + s * v_str[2];
          for (int64_t c = 0; c < d; ++c) acc[c] += w * bf16_to_double(vrow[c]);
        }
      }
      for (int64_t c = 0; c < d; ++c) out[i * d + c] = Z > 0.0 ? acc[c] / Z : 0.0;
      if (lse) lse[i] = Z > 0.0 ? m + log(Z) : -INFINITY;
    }
    free(x);
    free(allowed);
    free(present);
    free(bias);
    free(qv);
    free(acc);
  }
  free(pos_q);
  free(pos_k);
  return bad ? OR_ERR_ARG : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* allowed-pair count                                                        */
/* ------------------------------------------------------------------------ */
/* Counts (query token, key token) pairs that take part: both real (index <
 * N), the key block listed for the query's block row, and s <= t when causal
 * (positions are the unpermuted ones; causal is only defined without a
 * permutation). Token-by-token loop. */
int64_t oracle_count_pairs(const int32_t *row_ptr, const int32_t *col, int64_t R, int64_t N,
                           int64_t block, int causal) {
  if (!row_ptr || !col || R < 0 || N <= 0 || block <= 0) return OR_ERR_ARG;
  int64_t nQB = (N + block - 1) / block, total = 0;
#pragma omp parallel for reduction(+ : total) schedule(dynamic, 8)
  for (int64_t r = 0; r < R; ++r) {
    int64_t u = r % nQB;
    for (int32_t e = row_ptr[r]; e < row_ptr[r + 1]; ++e) {
      int64_t vb = col[e];
      for (int64_t t = u * block; t < (u + 1) * block && t < N; ++t)
        for (int64_t s = vb * block; s < (vb + 1) * block && s < N; ++s)
          if (!causal || s <= t) ++total;
    }
  }
  return total;
}


/* ------------------------------------------------------------------------ */
/* centroids: segment offsets and segment means                              */
/* ------------------------------------------------------------------------ */
/* seg_ptr[bh][g] = number of tokens of head bh whose label is in [0, g), for
 * g = 0..G (labels outside [0, G) are not counted: they sort after every
 * valid label).  seg_ptr is [BH][G + 1]. */
int oracle_segment_offsets(const int32_t *labels, int64_t BH, int64_t N, int32_t G, int32_t *seg_ptr) {
  if (!labels || !seg_ptr || BH < 0 || N < 0 || G <= 0) return OR_ERR_ARG;
  for (int64_t bh = 0; bh < BH; ++bh) {
    int32_t *sp = seg_ptr + bh * (G + 1);
    for (int32_t g = 0; g <= G; ++g) sp[g] = 0;
    for (int64_t t = 0; t < N; ++t) {
      int32_t l = labels[bh * N + t];
      if (l >= 0 && l < G) sp[l + 1] += 1;
    }
    for (int32_t g = 0; g < G; ++g) sp[g + 1] += sp[g];
  }
  return OR_OK;
}

/* means[bh][s][:] = mean of the bf16 rows x[b][h][i][:] for i in segment s of
 * head bh = (b, h): [seg_ptr[bh][s], seg_ptr[bh][s+1]) when seg_ptr != NULL,
 * else [s * seg_len, min(N, (s+1) * seg_len)) with G = ceil(N / seg_len).
 * Sums in fp64 in ascending i; an empty segment has mean 0.  xs: element
 * strides (batch, head, token). */
int oracle_segment_means(const uint16_t *x, const int64_t *xs, int64_t B, int64_t H, int64_t N, int64_t d,
                         const int32_t *seg_ptr, int32_t G, int32_t seg_len, float *means) {
  if (!x || !xs || !means || B < 0 || H < 0 || N < 0 || d <= 0 || G <= 0) return OR_ERR_ARG;
  if (!seg_ptr && seg_len <= 0) return OR_ERR_ARG;
  double *acc = (double *)malloc(sizeof(double) * (size_t)d);
  if (!acc) return OR_ERR_ARG;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h) {
      int64_t bh = b * H + h;
      for (int32_t s = 0; s < G; ++s) {
        int64_t lo, hi;
        if (seg_ptr) {
          lo = seg_ptr[bh * (G + 1) + s];
          hi = seg_ptr[bh * (G + 1) + s + 1];
        } else {
          lo = (int64_t)s * seg_len;
          hi = lo + seg_len < N ? lo + seg_len : N;
        }
        for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
        for (int64_t i = lo; i < hi; ++i)
          for (int64_t c = 0; c < d; ++c) acc[c] += bf16_to_double(x[b * xs[0] + h * xs[1] + i * xs[2] + c]);
        float *m = means + (bh * G + s) * d;
        for (int64_t c = 0; c < d; ++c) m[c] = hi > lo ? (float)(acc[c] / (double)(hi - lo)) : 0.0f;
      }
    }
  free(acc);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* group-shared importance sampling over KV tiles                            */
/* ------------------------------------------------------------------------ */
typedef struct {
  double mass;
  int32_t v;
} tile_mass;

static int cmp_mass_desc(const void *a, const void *b) {
  const tile_mass *x = (const tile_mass *)a, *y = (const tile_mass *)b;
  if (x->mass != y->mass) return x->mass > y->mass ? -1 : 1;
  return x->v < y->v ? -1 : (x->v > y->v);
}

/* For every head (b, h) and query group g (the query blocks u whose first
 * token, u * block, lies in segment g of q_seg_ptr):
 *   score:    a_v = scale * qbar[bh][g] . kbar[(b, h / (Hq/Hkv))][v], summed
 *             in fp64 over ascending components; the tile's mass is
 *             |v| * exp(a_v - max_v a_v), |v| its number of real keys (the
 *             size x centroid-score product of step 4; the common factor
 *             exp(-max) cancels in every step below);
 *   exact:    the m_exact tiles of largest mass, ties to the lower v;
 *   residual: the other tiles; pi = min(1, lam * mass) with sum m_sample
 *             (Eq. 4), or pi = 1 for all when there are at most m_sample;
 *   sample:   systematic PPS over the residual in ascending v: the points
 *             u0 + k, k = 0..m_sample-1, u0 = uoff[bh][g] in [0, 1), fall
 *             in the intervals [c_v, c_v + pi_v) of the running sum c;
 *   weights:  exact and sampled tiles are kept; a sampled tile with pi < 1
 *             gets lw = -ln(pi) (w = 1/pi, step 13), every other kept tile
 *             and the diagonal tile lw = 0.
 * mask/lw_map rows r = bh * nQB + u, [R][nKB], written in full (rows with no
 * group are all zero).  pi_out (optional, [BH][G][nKB]): pi of residual
 * tiles, 1 for exact tiles, 0 for groups with no query block. */
int oracle_is_sample(const float *qbar, const float *kbar, const int32_t *q_seg_ptr, const double *uoff,
                     int64_t B, int64_t Hq, int64_t Hkv, int32_t G, int64_t N, int32_t block, int64_t d,
                     int32_t m_exact, int32_t m_sample, double scale, uint8_t *mask, float *lw_map,
                     double *pi_out) {
  if (!qbar || !kbar || !q_seg_ptr || !uoff || !mask || !lw_map) return OR_ERR_ARG;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || G <= 0 || N <= 0 || block <= 0 || d <= 0) return OR_ERR_ARG;
  if (m_exact < 0 || m_sample < 0) return OR_ERR_ARG;
  int64_t nb = (N + block - 1) / block;
  memset(mask, 0, (size_t)(B * Hq * nb * nb));
  memset(lw_map, 0, sizeof(float) * (size_t)(B * Hq * nb * nb));
  if (pi_out) memset(pi_out, 0, sizeof(double) * (size_t)(B * Hq * G * nb));
  double *a = (double *)malloc(sizeof(double) * (size_t)nb);
  double *pi = (double *)malloc(sizeof(double) * (size_t)nb);
  uint8_t *keep = (uint8_t *)malloc((size_t)nb);
  uint8_t *exact = (uint8_t *)malloc((size_t)nb);
  tile_mass *tm = (tile_mass *)malloc(sizeof(tile_mass) * (size_t)nb);
  int rc = OR_OK;
  if (!a || !pi || !keep || !exact || !tm) rc = OR_ERR_ARG;
  for (int64_t bh = 0; rc == OR_OK && bh < B * Hq; ++bh) {
    int64_t b = bh / Hq, h = bh % Hq, gk = b * Hkv + h / (Hq / Hkv);
    for (int32_t g = 0; g < G; ++g) {
      int64_t s0 = q_seg_ptr[bh * (G + 1) + g], s1 = q_seg_ptr[bh * (G + 1) + g + 1];
      int64_t u0 = (s0 + block - 1) / block, u1 = (s1 + block - 1) / block;   /* u * block in [s0, s1) */
      if (u1 > nb) u1 = nb;
      if (u0 >= u1) continue;
      /* step 2: centroid scores, and the tile masses */
      const float *qg = qbar + (bh * G + g) * d;
      double amax = -INFINITY;
      for (int64_t v = 0; v < nb; ++v) {
        const float *kv = kbar + (gk * nb + v) * d;
        double s = 0.0;
        for (int64_t c = 0; c < d; ++c) s += (double)qg[c] * (double)kv[c];
        a[v] = scale * s;
        if (a[v] > amax) amax = a[v];
      }
      for (int64_t v = 0; v < nb; ++v) {
        int64_t size = N - v * block < block ? N - v * block : block;
        tm[v].mass = (double)size * exp(a[v] - amax);
        tm[v].v = (int32_t)v;
      }
      /* step 4: exact set */
      qsort(tm, (size_t)nb, sizeof(tile_mass), cmp_mass_desc);
      memset(exact, 0, (size_t)nb);
      int64_t ne = m_exact < nb ? m_exact : nb;
      for (int64_t i = 0; i < ne; ++i) exact[tm[i].v] = 1;
      /* step 10: inclusion probabilities of the residual (tm[ne..nb) is the
       * residual in descending mass) */
      int64_t nr = nb - ne;
      for (int64_t v = 0; v < nb; ++v) pi[v] = exact[v] ? 1.0 : 0.0;
      if (nr <= m_sample) {
        for (int64_t i = ne; i < nb; ++i) pi[tm[i].v] = 1.0;
      } else {
        /* suffix sums of the residual masses, from the smallest up */
        double *suf = a; /* reuse: a is no longer needed */
        double run = 0.0;
        for (int64_t i = nb - 1; i >= ne; --i) {
          run += tm[i].mass;
          suf[i] = run;
        }
        /* the number k of capped tiles: the smallest k for which the k-th
         * largest residual mass is not capped by lam_k = (m - k) / suf */
        int64_t k = 0;
        while (k < m_sample && (double)(m_sample - k) * tm[ne + k].mass > suf[ne + k]) ++k;
        double lam = (double)(m_sample - k) / suf[ne + k];
        for (int64_t i = 0; i < nr; ++i) pi[tm[ne + i].v] = i < k ? 1.0 : lam * tm[ne + i].mass;
      }
      /* step 11: systematic PPS over the residual in ascending v */
      memset(keep, 0, (size_t)nb);
      double c = 0.0, u = uoff[bh * G + g];
      for (int64_t v = 0; v < nb; ++v) {
        if (exact[v]) {
          keep[v] = 1;
          continue;
        }
        double lo = c;
        c += pi[v];
        double klo = ceil(lo - u), khi = ceil(c - u);
        if (klo > m_sample) klo = m_sample;
        if (khi > m_sample) khi = m_sample;
        if (khi > klo) keep[v] = 1;
      }
      /* step 13: weights; rows of the group */
      for (int64_t uq = u0; uq < u1; ++uq) {
        int64_t r = bh * nb + uq;
        for (int64_t v = 0; v < nb; ++v) {
          if (!keep[v]) continue;
          mask[r * nb + v] = 1;
          lw_map[r * nb + v] = (!exact[v] && pi[v] < 1.0 && v != uq) ? (float)(-log(pi[v])) : 0.0f;
        }
      }
      if (pi_out)
        for (int64_t v = 0; v < nb; ++v) pi_out[(bh * G + g) * nb + v] = pi[v];
    }
  }
  free(a);
  free(pi);
  free(keep);
  free(exact);
  free(tm);
  return rc;
}


/* ------------------------------------------------------------------------ */
/* token-level attention over computational query sets                      */
/* ------------------------------------------------------------------------ */
/* CQS c of head bh = b*Hq + h: query positions q_idx[(bh*C + c)*BQ + i]
 * (i < BQ; a position outside [0, N) is an empty slot) and key positions
 * kv_idx[kv_ptr[bh*C + c] .. kv_ptr[bh*C + c + 1]).  For each requested slot
 * (slots[j] = (bh*C + c)*BQ + i): O = sum_e softmax_e(x_e) V[s_e] over the
 * list entries e with s_e in [0, N) and, when causal, s_e <= t, with
 * x_e = scale * Q[t] . K[s_e] (K and V of head b*Hkv + h/(Hq/Hkv));
 * LSE = ln sum_e exp(x_e).  No allowed entry: O = 0, LSE = -inf.  An empty
 * slot gives O = 0 and LSE = NaN. */
int oracle_attn_tok(const uint16_t *q, const uint16_t *k, const uint16_t *v, const int64_t *q_str,
                    const int64_t *k_str, const int64_t *v_str, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                    int64_t d, int64_t C, int64_t BQ, const int32_t *q_idx, const int32_t *kv_ptr,
                    const int32_t *kv_idx, int causal, double scale, int64_t n_slots, const int64_t *slots,
                    double *out, double *lse) {
  if (!q || !k || !v || !q_idx || !kv_ptr || !kv_idx || !slots || !out || !lse) return OR_ERR_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N <= 0 || d <= 0 || C <= 0 || BQ <= 0) return OR_ERR_ARG;
  int64_t G = Hq / Hkv;
  int bad = 0;
#pragma omp parallel
  {
    double *qv = (double *)malloc(sizeof(double) * (size_t)d);
    double *acc = (double *)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 16)
    for (int64_t j = 0; j < n_slots; ++j) {
      int64_t slot = slots[j];
      int64_t cq = slot / BQ;
      if (slot < 0 || cq >= B * Hq * C) {
        bad = 1;
        continue;
      }
      int64_t bh = cq / C, b = bh / Hq, h = bh % Hq, g = h / G;
      int64_t t = q_idx[slot];
      for (int64_t c = 0; c < d; ++c) out[j * d + c] = 0.0;
      if (t < 0 || t >= N) {
        lse[j] = NAN;
        continue;
      }
      const uint16_t *qrow = q + b * q_str[0] + h * q_str[1] + t * q_str[2];
      for (int64_t c = 0; c < d; ++c) qv[c] = bf16_to_double(qrow[c]);
      int32_t e0 = kv_ptr[cq], e1 = kv_ptr[cq + 1];
      double m = -INFINITY;
      for (int32_t e = e0; e < e1; ++e) {
        int64_t s = kv_idx[e];
        if (s < 0 || s >= N || (causal && s > t)) continue;
        const uint16_t *krow = k + b * k_str[0] + g * k_str[1] + s * k_str[2];
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qv[c] * bf16_to_double(krow[c]);
        if (scale * dot > m) m = scale * dot;
      }
      double Z = 0.0;
      for (int64_t c = 0; c < d; ++c) acc[c] = 0.0;
      if (m != -INFINITY) {
        for (int32_t e = e0; e < e1; ++e) {
          int64_t s = kv_idx[e];
          if (s < 0 || s >= N || (causal && s > t)) continue;
          const uint16_t *krow = k + b * k_str[0] + g * k_str[1] + s * k_str[2];
          double dot = 0.0;
          for (int64_t c = 0; c < d; ++c) dot += qv[c] * bf16_to_double(krow[c]);
          double w = exp(scale * dot - m);
          Z += w;
          const uint16_t *vrow = v + b * v_str[0] + g * v_str[1] + s * v_str[2];
          for (int64_t c = 0; c < d; ++c) acc[c] += w * bf16_to_double(vrow[c]);
        }
      }
      for (int64_t c = 0; c < d; ++c) out[j * d + c] = Z > 0.0 ? acc[c] / Z : 0.0;
      lse[j] = Z > 0.0 ? m + log(Z) : -INFINITY;
    }
    free(qv);
    free(acc);
  }
  return bad ? OR_ERR_ARG : OR_OK;
}

/* ------------------------------------------------------------------------ */
/* MC-Sparse exact token selection                                          */
/* ------------------------------------------------------------------------ */
/* Group mass (MC-Sparse, implementation details: a first dense pass gives
 * each query's log-sum-exp, a second recomputes the scores, recovers the
 * probabilities and aggregates them per query group).  For group c of head
 * bh (query positions q_idx[(bh*C + c)*BQ + i], a position outside [0, N)
 * being an empty slot) and key s in [s0, s1):
 *   mass = sum over the group's queries t (s <= t when causal) of
 *          exp(x_ts - LSE_t),  x_ts = scale * Q[t] . K[s],
 *   LSE_t = ln sum over all keys s' of the query (s' <= t when causal) of
 *           exp(x_ts').
 * Output mass[(bh*C + c)*(s1 - s0) + (s - s0)], fp64. */
int oracle_group_mass(const uint16_t *q, const uint16_t *k, const int64_t *q_str, const int64_t *k_str, int64_t B,
                      int64_t Hq, int64_t Hkv, int64_t N, int64_t d, int64_t C, int64_t BQ, const int32_t *q_idx,
                      int causal, double scale, int64_t s0, int64_t s1, double *mass) {
  if (!q || !k || !q_idx || !mass) return OR_ERR_ARG;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N <= 0 || d <= 0 || C <= 0 || BQ <= 0) return OR_ERR_ARG;
  if (s0 < 0 || s1 > N || s0 > s1) return OR_ERR_ARG;
  int64_t G = Hq / Hkv, W = s1 - s0;
#pragma omp parallel
  {
    double *qv = (double *)malloc(sizeof(double) * (size_t)d);
    double *x = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t cq = 0; cq < B * Hq * C; ++cq) {
      int64_t bh = cq / C, b = bh / Hq, h = bh % Hq, g = h / G;
      double *out = mass + cq * W;
      for (int64_t s = 0; s < W; ++s) out[s] = 0.0;
      for (int64_t i = 0; i < BQ; ++i) {
        int64_t t = q_idx[cq * BQ + i];
        if (t < 0 || t >= N) continue;
        const uint16_t *qrow = q + b * q_str[0] + h * q_str[1] + t * q_str[2];
        for (int64_t c = 0; c < d; ++c) qv[c] = bf16_to_double(qrow[c]);
        int64_t smax = causal ? t + 1 : N;   /* keys [0, smax) take part */
        double m = -INFINITY;
        for (int64_t s = 0; s < smax; ++s) {
          const uint16_t *krow = k + b * k_str[0] + g * k_str[1] + s * k_str[2];
          double dot = 0.0;
          for (int64_t c = 0; c < d; ++c) dot += qv[c] * bf16_to_double(krow[c]);
          x[s] = scale * dot;
          if (x[s] > m) m = x[s];
        }
        double Z = 0.0;
        for (int64_t s = 0; s < smax; ++s) Z += exp(x[s] - m);
        double lse = m + log(Z);
        for (int64_t s = s0; s < s1 && s < smax; ++s) out[s - s0] += exp(x[s] - lse);
      }
    }
    free(qv);
    free(x);
  }
  return OR_OK;
}

/* The K largest of each row of mass[rows][N] (MC-Sparse: top-K on the
 * aggregated attention mass), ties broken toward the lower index; written
 * to idx[rows][min(K, N)] in ascending index order. */
static const double *topk_base;
static int topk_cmp(const void *a, const void *b) {
  int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
  double x = topk_base[i], y = topk_base[j];
  if (x > y) return -1;
  if (x < y) return 1;
  return (i > j) - (i < j);
}
static int asc_cmp(const void *a, const void *b) {
  int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
  return (i > j) - (i < j);
}
int oracle_topk(const double *mass, int64_t rows, int64_t N, int64_t K, int32_t *idx) {
  if (!mass || !idx || rows < 0 || N <= 0 || K < 0) return OR_ERR_ARG;
  int64_t k = K < N ? K : N;
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
  if (!order) return OR_ERR_ARG;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t s = 0; s < N; ++s) order[s] = (int32_t)s;
    topk_base = mass + r * N;   /* single-threaded: qsort has no context argument */
    qsort(order, (size_t)N, sizeof(int32_t), topk_cmp);
    qsort(order, (size_t)k, sizeof(int32_t), asc_cmp);
    memcpy(idx + r * k, order, sizeof(int32_t) * (size_t)k);
  }
  free(order);
  return OR_OK;
}
