/*
 * bsattn.h -- block-sparse (optionally permuted) softmax attention forward on
 * AMD Instinct MI355X (gfx950).  C ABI of libbsattn.so.
 *
 * Terminology
 *   B, Hq, Hkv, N, d   batch, query heads, key/value heads (Hq % Hkv == 0),
 *                      tokens, head dimension.
 *   block              query block size = key block size (64 or 128).
 *   nQB = nKB          ceil(N / block); the last block may be partial.
 *   row                one (batch, query head, query block) triple,
 *                      r = (b * Hq + h) * nQB + u, R = B * Hq * nQB rows.
 *   CSR                row_ptr[R + 1] (int32) and col[nnz] (int32, ascending
 *                      KV-block indices per row), optional lw[nnz] (float32
 *                      additive log-weight of each listed block).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument that names device memory must be device memory
 *     allocated by the caller; the library never allocates or frees device
 *     memory and keeps no state between calls.
 *   - Work is enqueued on the caller's HIP stream and is asynchronous, except
 *     bsa_csr_count, which synchronises the stream to return nnz.
 *   - Return value: BSA_OK (0) or a negative BSA_ERR_* code.  Argument checks
 *     run on the host before any HIP call; on an argument error nothing is
 *     enqueued.  BSA_ERR_HIP reports a failed launch or HIP runtime call.
 *   - Token-major tensors are addressed with int64 element strides for
 *     (batch, head, token); the head dimension must be contiguous, base
 *     pointers 16-byte aligned and strides multiples of 8 elements.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSA_OK 0
#define BSA_ERR_ARG (-1)         /* null pointer, bad size, stride or alignment */
#define BSA_ERR_UNSUPPORTED (-2) /* d or block not in {64,128}, causal with a permutation, size limits */
#define BSA_ERR_HIP (-4)         /* HIP runtime or launch failure */

typedef void *bsa_stream_t; /* a hipStream_t; NULL is the default stream */

/* Layout of V for bsa_attn_fwd. */
#define BSA_V_TOKEN_MAJOR 0 /* [B][Hkv][N][d]: strides (batch, head, token), d contiguous */
#define BSA_V_DIM_MAJOR 1   /* [B][Hkv][d][ld]: strides (batch, head, dim row), keys contiguous */

/* Library version, (major << 16) | minor. */
int bsa_version(void);

/* Static description of an error code (never NULL). */
const char *bsa_strerror(int code);

/* ---------------------------------------------------------------------------
 * Mask -> CSR, pass 1.
 *
 * Source: ScalingAttention (section 5.2, Eq. 2) instantiates the block mask of
 * density p from a threshold map as M_p = I(T <= p); the block-sparse mask of
 * WaveAlign (section II-B) has one row per query block whose retained entries
 * are the executed (query block, KV block) interactions.
 *
 * Entry (r, v) is kept when mask[r * nKB + v] != 0 (if mask != NULL), else
 * when T[r * nKB + v] <= p (float32 comparison; NaN is never kept), or when
 * force_diag != 0 and v == r % nQB (the diagonal block, so that no row is
 * empty).  Exactly one of mask (uint8, device) and T (float32, device) must be
 * non-NULL; both are [R][nKB] row-major.
 *
 * Writes row_ptr[0..R] (device, int32, caller-owned, R + 1 entries).  When
 * nnz_out != NULL, stores nnz = row_ptr[R] into *nnz_out (host) and
 * synchronises `stream`; with nnz_out == NULL the call is asynchronous (a
 * caller that sizes col by the bound R * nKB needs no host round trip).
 * Errors: BSA_ERR_ARG for NULL/negative sizes or both/neither sources;
 * BSA_ERR_UNSUPPORTED when R * nKB >= 2^31 or force_diag with nQB > nKB.
 * ------------------------------------------------------------------------- */
int bsa_csr_count(const uint8_t *mask, const float *T, float p, int64_t R, int32_t nQB,
                  int32_t nKB, int force_diag, int32_t *row_ptr, int64_t *nnz_out,
                  bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Mask -> CSR, pass 2.  Same keep rule and arguments as bsa_csr_count, with
 * row_ptr as it produced.  Writes col[row_ptr[r] ..] = kept v of row r in
 * ascending order (the order of the CRM forward iterator of ScalingAttention,
 * section 7.3, Algorithm 2).  When lw != NULL also writes lw[e] = the bits of
 * lw_map[r * nKB + v] (float32 [R][nKB], device), or 0.0f when lw_map is
 * NULL.  `capacity` is the number of entries col (and lw) can hold and
 * should be the nnz bsa_csr_count returned; entries at an index >= capacity
 * are never written (the list is truncated, nothing faults).  BSA_ERR_ARG for
 * capacity < 0 or col == NULL with capacity > 0.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_csr_fill(const uint8_t *mask, const float *T, float p, const float *lw_map, int64_t R,
                 int32_t nQB, int32_t nKB, int force_diag, const int32_t *row_ptr, int32_t *col,
                 float *lw, int64_t capacity, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Mask -> CRM rows.
 *
 * Source: ScalingAttention, section 7.2 (Compressed Row Mask: each row is an
 * aligned array of uint32 words, one bit per KV block, so one word load
 * decodes 32 block states).
 *
 * Same keep rule and mask/T/p/force_diag arguments as bsa_csr_count.  Writes
 * crm[r * W + v / 32] bit (v % 32) = 1 when entry (r, v) is kept, with
 * W = ceil(nKB / 32); bits for v >= nKB are written as 0.  crm: device
 * uint32 [R][W], caller-owned.  Errors as bsa_csr_count (crm == NULL is
 * BSA_ERR_ARG).  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_crm_build(const uint8_t *mask, const float *T, float p, int64_t R, int32_t nQB, int32_t nKB,
                  int force_diag, uint32_t *crm, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * CRM rows -> CSR row offsets: row_ptr[0] = 0, row_ptr[r + 1] = row_ptr[r] +
 * popcount of row r (bits for v >= nKB are ignored).  crm: device uint32
 * [R][ceil(nKB / 32)]; row_ptr: device int32 [R + 1] (output).  When
 * nnz_out != NULL, stores row_ptr[R] there (host) and synchronises `stream`;
 * otherwise asynchronous.  BSA_ERR_ARG for NULL pointers or negative sizes,
 * BSA_ERR_UNSUPPORTED when R * nKB >= 2^31.
 * ------------------------------------------------------------------------- */
int bsa_crm_row_ptr(const uint32_t *crm, int64_t R, int32_t nKB, int32_t *row_ptr, int64_t *nnz_out,
                    bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * CRM rows -> CSR column lists by the forward iterator of ScalingAttention,
 * section 7.3 (Algorithm 2: ascending walk by count-trailing-zeros and
 * clear-lowest-bit).  row_ptr as bsa_crm_row_ptr produced it; writes
 * col[row_ptr[r] ..] = the blocks of row r in ascending order.  Entries at an
 * index >= capacity are never written.  BSA_ERR_ARG for NULL pointers,
 * negative sizes or capacity < 0.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_crm_to_csr(const uint32_t *crm, int64_t R, int32_t nKB, const int32_t *row_ptr, int32_t *col,
                   int64_t capacity, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Cluster labels -> gather permutation.
 *
 * Source: permuted block-sparse attention clusters queries and keys and
 * permutes the tokens so that every cluster is contiguous (InstaGen,
 * section 4; WaveAlign, section IV-A: rows are permuted and outputs
 * restored).
 *
 * labels: int32 [BH][N] (device).  perm: int32 [BH][N] (device, output):
 * perm[bh][i] is the original index of the token placed at position i; the
 * order is ascending (label, original index), so equal labels keep their
 * original order.  Labels outside [0, n_clusters) sort after all valid
 * labels.  n_clusters must be in [1, 4095].  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_perm_from_labels(const int32_t *labels, int64_t BH, int64_t N, int32_t n_clusters,
                         int32_t *perm, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Row gather / scatter of a [B][H][N][d] bf16 tensor by a per-(b,h)
 * permutation perm [B*H][N] (device, int32, gather form as above).
 *   bsa_permute_rows:   dst[b][h][i]       = src[b][h][perm[bh][i]]
 *   bsa_unpermute_rows: dst[b][h][perm[bh][i]] = src[b][h][i]
 * (WaveAlign, section V: permute query rows before attention and restore the
 * output order after it.)  src and dst are bf16 (uint16 bits), strides in
 * elements for (batch, head, token); d in {64, 128}; src and dst must not
 * overlap.  An index outside [0, N) is skipped (gather writes zeros).
 * Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_permute_rows(const void *src, void *dst, const int32_t *perm, int32_t B, int32_t H,
                     int64_t N, int32_t d, const int64_t src_strides[3],
                     const int64_t dst_strides[3], bsa_stream_t stream);
int bsa_unpermute_rows(const void *src, void *dst, const int32_t *perm, int32_t B, int32_t H,
                       int64_t N, int32_t d, const int64_t src_strides[3],
                       const int64_t dst_strides[3], bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Gather + transpose into the dim-major layout bsa_attn_fwd reads fastest.
 *   dst[b][h][c][i] = src[b][h][perm ? perm[bh][i] : i][c]   for i < N
 *   dst[b][h][c][i] = 0                                       for N <= i < ld
 * (the V side of the permutation step of permuted block-sparse attention,
 * written key-contiguous so that the attention kernel's P.V contraction reads
 * 16-byte rows).  src: bf16 [B][H][N][d], strides (batch, head, token), d
 * contiguous.  dst: bf16, strides (batch, head, dim row), keys contiguous;
 * dst_strides[2] >= ld; ld >= N and a multiple of 8; d in {64, 128}.
 * perm (int32 [B*H][N], device) may be NULL.  An index outside [0, N) in perm
 * gathers zeros.  src and dst must not overlap.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_transpose_rows(const void *src, void *dst, const int32_t *perm, int32_t B, int32_t H,
                       int64_t N, int32_t d, int64_t ld, const int64_t src_strides[3],
                       const int64_t dst_strides[3], bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * WaveAlign stage 1: polar spectral order of each head's query blocks.
 *
 * Source: WaveAlign, section IV-C (C.1 polar spectral ordering of a rank-2
 * embedding of the mask rows; C.2 matrix-free centred subspace iteration).
 *
 * For every head h in [0, BH) (CSR rows h*nQB .. h*nQB + nQB - 1): the
 * nQB x nKB 0/1 block mask M is centred, C = M - 1 mu^T with mu the column
 * means; `iters` steps of X <- orth(C C^T X) (Gram-Schmidt, start
 * X0[u] = (((37u + 11) mod 101)/101 - 1/2, ((53u + 29) mod 97)/97 - 1/2))
 * give rank-2 row coordinates, and rows are ordered by their polar angle
 * atan2(X[u][1], X[u][0]), ties by u.  fp64 throughout.
 * row_ptr: device int32 [BH*nQB + 1]; col: device int32 [nnz] (entries
 * outside [0, nKB) are ignored).  perm: device int32 [BH][nQB] (output):
 * perm[h][p] = query block at position p, a permutation of 0..nQB-1 per head.
 * angle: device float64 [BH][nQB] (output, may be NULL): the angle of each
 * query block.  enable: device int32 [1] or NULL; when it is given and holds
 * 0 (the adaptive skip's decision, bsa_stage1_decide) the order is not
 * computed: perm is the identity and angle (when given) is 0, so a schedule
 * built from it equals the one built without a stage-1 order.  nQB, nKB <=
 * 1024, nKB * ceil(nQB / 32) <= 12288 and nQB * ceil(nKB / 32) <= 12288
 * (e.g. 614 x 614 or 512 x 768), else BSA_ERR_UNSUPPORTED; iters >= 1.
 * Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_spectral_order(const int32_t *row_ptr, const int32_t *col, int32_t BH, int32_t nQB, int32_t nKB,
                       int32_t iters, int32_t *perm, double *angle, const int32_t *enable,
                       bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * WaveAlign adaptive skip: should stage 1 run for these lists?
 *
 * Source: WaveAlign, section IV-E (Runtime Coordination: the skip module
 * bypasses the reordering when its estimated latency reduction does not
 * exceed its overhead) and section VI-F with Figure 13 (skipped at low
 * retained densities, enabled from 14.5 %).  The pages state the rule in
 * words; this estimate is the library's reading of it, computed on the
 * device so that no host round trip is needed.
 *
 * Over the BH heads' CSR rows (row_ptr device int32 [BH*nQB + 1], col device
 * int32, every row ascending as bsa_csr_fill writes them; for other lists
 * fresh is unspecified): nnz = listed entries (each is one tile the
 * attention kernels process), nmax = the largest per-head nnz, fresh =
 * entries a row lists whose block the previous row of its head does not
 * list (all of the first row's).  With f = fresh/nnz, density = nnz/(BH nQB nKB),
 * t_attn = nnz tile_ms (block/128)^2 (d/128) / n_cus (ms), gain = gamma f
 * t_attn, cost = (iters/10)(row_ms nQB + nnz_ms nmax) (ms): stage 1 runs when
 * 4 N d (bytes of K and V of a head) > l2_bytes, density >= density_min,
 * gain > cost, and bsa_spectral_order supports (nQB, nKB).
 * params: host pointer or NULL for the defaults (bsa_stage1_default_params:
 * gamma 0.04, tile_ms 2.1e-3, row_ms 8.6e-4, nnz_ms 3.5e-6, density_min
 * 0.10, l2_bytes 4 MiB, measured on MI355X).  decision: device int32 [1]
 * (output, 0 or 1).  stats: device float64 [7] (output, may be NULL): f,
 * density, t_attn, gain, cost, K/V bytes per head, decision.
 * BSA_ERR_ARG for NULL pointers or non-positive sizes / iters / n_cus;
 * BSA_ERR_UNSUPPORTED for BH*nQB >= 2^31.  Asynchronous (three launches: the
 * fresh count is an integer sum over one wavefront per row, so the
 * statistics do not depend on timing; decision[0] holds that count until
 * the last launch overwrites it with the decision).
 * ------------------------------------------------------------------------- */
typedef struct {
  double gamma, tile_ms, row_ms, nnz_ms, density_min, l2_bytes;
} bsa_stage1_params;

void bsa_stage1_default_params(bsa_stage1_params *params);
int bsa_stage1_decide(const int32_t *row_ptr, const int32_t *col, int32_t BH, int32_t nQB, int32_t nKB, int64_t N,
                      int32_t d, int32_t block, int32_t iters, int32_t n_cus, const bsa_stage1_params *params,
                      int32_t *decision, double *stats, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Segment offsets of labelled tokens (centroid groups).
 *
 * Source: InstaGen, Algorithm 1 step 1 and section 4 (queries and keys are
 * grouped by cluster label and permuted into contiguous blocks); the tokens
 * of label g occupy one segment of the label-sorted sequence (the order
 * bsa_perm_from_labels produces).
 *
 * labels: device int32 [BH][N].  seg_ptr: device int32 [BH][G + 1] (output):
 * seg_ptr[bh][g] = number of tokens of head bh with a label in [0, g); labels
 * outside [0, G) are not counted (they sort after every valid label).
 * BSA_ERR_ARG for NULL pointers, negative sizes or G <= 0;
 * BSA_ERR_UNSUPPORTED for G > 8192 or N >= 2^31.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_segment_offsets(const int32_t *labels, int64_t BH, int64_t N, int32_t G, int32_t *seg_ptr,
                        bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Segment means (centroids).
 *
 * Source: InstaGen, Algorithm 1 step 2 (the centroid of a query group and of
 * a key cluster); at tile granularity the key cluster of a KV tile is the
 * tile itself, with its mean key as centroid.
 *
 * x: bf16 [B][H][N][d] (device, element strides x_str: batch, head, token;
 * d contiguous; 16-byte aligned base, strides multiples of 8).  Segment s of
 * head bh = b*H + h is rows [seg_ptr[bh][s], seg_ptr[bh][s+1]) when seg_ptr
 * != NULL (device int32 [BH][G + 1], e.g. from bsa_segment_offsets over the
 * label-sorted rows), else rows [s*seg_len, min(N, (s+1)*seg_len)) with
 * G = ceil(N / seg_len) segments.  means: device float32 [BH][G][d]
 * (output): the fp32 mean of the segment's rows, 0 for an empty segment.
 * BSA_ERR_ARG for NULL pointers, non-positive sizes, misaligned strides;
 * BSA_ERR_UNSUPPORTED for d % 8 != 0, d > 256, a misaligned x or
 * B*H > 65535.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_segment_means(const void *x, const int64_t x_str[3], int32_t B, int32_t H, int64_t N, int32_t d,
                      const int32_t *seg_ptr, int32_t G, int32_t seg_len, float *means, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Group-shared importance sampling over KV tiles.
 *
 * Source: InstaGen, Algorithm 1 steps 2-13, section 3.2.1 Eq. (4) and the
 * systematic PPS sample of section 4, at tile granularity (each 128-key tile
 * is entirely exact or entirely sampled; weights enter as a logit bias).
 *
 * For every head bh = b*Hq + h and query group g (the query blocks u whose
 * first token u*block lies in segment g of q_seg_ptr):
 *   - a_v = scale * qbar[bh][g] . kbar[b*Hkv + h/(Hq/Hkv)][v] (fp64), and
 *     the tile mass |v| exp(a_v - max a), |v| = real keys of tile v;
 *   - exact set: the m_exact tiles of largest mass (ties to the lower v);
 *   - residual: pi_v = min(1, lam * mass_v) with sum m_sample (Eq. 4), or 1
 *     for every residual tile when there are at most m_sample;
 *   - sample: systematic PPS over the residual in ascending v with the points
 *     uoff[bh][g] + j, j = 0..m_sample-1 (uoff in [0, 1), drawn by the
 *     caller);
 *   - rows: mask[r][v] = 1 for exact and sampled tiles, lw_map[r][v] =
 *     -ln(pi_v) for sampled tiles with pi_v < 1, else 0 (0 on the diagonal
 *     v = u, which the CSR builder forces as exact).
 * Rows r = bh*nKB + u with no group are written as zeros; every row is
 * written.  The outputs feed bsa_csr_count / bsa_csr_fill (mask, lw_map,
 * force_diag = 1).
 *
 * qbar: device float32 [B*Hq][G][d]; kbar: device float32 [B*Hkv][nKB][d]
 * (nKB = ceil(N / block)); q_seg_ptr: device int32 [B*Hq][G + 1]; uoff:
 * device float64 [B*Hq][G]; mask: device uint8 [B*Hq*nKB][nKB]; lw_map:
 * device float32, same shape; pi_out: optional device float64
 * [B*Hq][G][nKB] (pi of every tile, 1 for exact tiles; 0 for groups without
 * a query block).  scale <= 0 selects 1/sqrt(d).  BSA_ERR_ARG for NULL
 * pointers, non-positive sizes, Hq % Hkv != 0 or negative budgets;
 * BSA_ERR_UNSUPPORTED for nKB > 1024, d > 256, G > 65535 or B*Hq > 65535.
 * Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_is_sample(const float *qbar, const float *kbar, const int32_t *q_seg_ptr, const double *uoff, int32_t B,
                  int32_t Hq, int32_t Hkv, int32_t G, int64_t N, int32_t block, int32_t d, int32_t m_exact,
                  int32_t m_sample, float scale, uint8_t *mask, float *lw_map, double *pi_out,
                  bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Row schedule (launch order of the attention kernel).
 *
 * Source: WaveAlign, section IV-D (rows in consecutive buckets of at most W,
 * each bucket sorted by descending nonzero-block count, long rows first) and
 * section VI-B (sequential-head scheduling).
 *
 * Logical sequence: for each batch b and KV head g, the rows of the
 * G = Hq / Hkv query heads sharing g, position p outer and head inner; the
 * row at position p of head h is query block p, or query block
 * row_perm[h][p] when a stage-1 order is given (row_perm: device int32
 * [B*Hq][nQB], a permutation of 0..nQB-1 per head, or NULL; an entry outside
 * [0, nQB) yields launch entry -1, which the attention kernel skips).
 * Buckets of `wave_rows` consecutive entries within each (b, g) segment are
 * sorted by (nnz descending, sequence position ascending).  When n_xcd > 1
 * the list is dealt to launch indices so that the GPU's round-robin dispatch
 * gives XCD x the x-th contiguous slice:
 * order[i] = logical[start(i % n_xcd) + i / n_xcd].  wave_rows = 0 selects
 * 2048 (a whole segment of up to 2048 rows is one bucket); then, when col
 * (the CSR block lists, device int32, optional) is given, each bucket keeps
 * the sorted order only if its consecutive rows share at least as many KV
 * blocks as in the sequence order (the rows an XCD runs one after another
 * reuse each other's K/V in L2), estimated with a 256-bit signature per row
 * (bit v mod 256 of every listed block v): the cost of an order is the sum
 * over its rows of the signature bits a row sets that the previous row does
 * not (the first row: all of them), and the sequence order is kept when its
 * cost is smaller.  head_step 1
 * schedules every row; head_step 2 only the rows of the first head of each
 * pair of query heads sharing a KV head (heads g*G + 2j), for the attention
 * path that serves a pair's identical rows in one launch (kv_share), and
 * needs G even.  row_ptr: device int32 [B*Hq*nQB + 1]; order: device int32
 * [B*Hq*nQB / head_step] (output).  wave_rows <= 2048.  BSA_ERR_ARG for
 * NULL pointers, non-positive sizes, Hq % Hkv != 0, head_step not 1 or 2 or
 * not dividing G.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_schedule(const int32_t *row_ptr, const int32_t *col, int32_t B, int32_t Hq, int32_t Hkv, int32_t nQB,
                 int32_t wave_rows, int32_t n_xcd, const int32_t *row_perm, int32_t head_step, int32_t *order,
                 bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Row schedule with identical rows paired (launch tables for bsa_attn_fwd's
 * order and order2).
 * Source: the buckets, their longest-first order and the XCD deal of
 * bsa_schedule (WaveAlign, section IV-D; head step 1); the pairing is the
 * library's reading of the schedule's purpose (WaveAlign, section IV: rows
 * that run together should reuse the same K/V blocks): two rows that list the
 * same blocks are served by one launch entry, which stages each K/V tile once
 * for both.  Within each bucket, walking its positions in ascending order, a
 * position that is not already the second row of a pair is paired with the
 * same head's next position (the next query block, or the next one of the
 * stage-1 order) when that position lies in the bucket and both rows list
 * the same blocks in the same order with the same log-weight bits (lw
 * optional).  Entries are keyed by their tile count (nnz, or 2 nnz for a
 * pair) and ordered as bsa_schedule orders rows (wave_rows 0: the sorted or
 * the position order per bucket by the same signature cost, taken over each
 * entry's first row); the second rows of pairs follow at the end of their
 * bucket as empty entries.  order[i] receives entry i's first row (-1 for an
 * empty entry), order2[i] its second row or -1.  row_ptr: device int32
 * [B*Hq*nQB + 1]; col, lw: device, as bsa_csr_fill writes them (col
 * required); row_perm: as bsa_schedule; order, order2: device int32
 * [B*Hq*nQB] (outputs; every row appears exactly once in them).
 * BSA_ERR_ARG for NULL pointers, non-positive sizes, Hq % Hkv != 0 or bad
 * wave_rows / n_xcd; BSA_ERR_UNSUPPORTED for wave_rows > 2048, Hq / Hkv >
 * 1024 or B*Hq*nQB >= 2^31.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_schedule_pairs(const int32_t *row_ptr, const int32_t *col, const float *lw, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t nQB, int32_t wave_rows, int32_t n_xcd, const int32_t *row_perm,
                       int32_t *order, int32_t *order2, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Block-sparse attention forward.
 *
 * Source: InstaGen, section 3.1 Eq. (1)-(3) (l_ij = q_i . k_j / sqrt(d),
 * o_i = sum_j softmax_j(l_ij) v_j) restricted to the KV blocks listed for the
 * query's block row (WaveAlign, section II-B), with the listed block's
 * log-weight added to the scaled logit (InstaGen, Algorithm 1: softmax of
 * l_ij + log w_j with Horvitz-Thompson weights).  Masked pairs contribute
 * nothing.  With causal != 0, key s is also masked for query t when s > t
 * (token positions; not allowed together with a permutation).  Keys and
 * queries at positions >= N in the last block do not take part.
 *
 * q [B][Hq][N][d], k [B][Hkv][N][d], o [B][Hq][N][d]: bf16 (uint16 bits)
 * device tensors addressed by the strides; query head h reads KV head
 * h / (Hq / Hkv).  v is bf16 in the layout v_layout names: BSA_V_DIM_MAJOR
 * (the fast path; dim-row stride v_str[2] >= ceil(N/block)*block, key columns
 * N.. of each row must hold finite values, e.g. the zeros bsa_transpose_rows
 * writes; per-head byte extents of q, k and v must stay below 2^30) or
 * BSA_V_TOKEN_MAJOR.  o must not alias q, k or v.  lse (float32 [B*Hq][N],
 * contiguous, device, optional) receives ln(sum_j exp(l_ij + log w_j)) of
 * every query.  row_ptr/col/lw: CSR as built above (lw optional); a block
 * index outside [0, nQB) in col takes no part (its keys are masked).  order
 * (optional, int32 [R]): launch index -> row; rows not listed are not
 * computed, nor is anything for an entry outside [0, R).  scatter_perm_q
 * (optional, int32 [B*Hq][N]): when set, the output of the query at position
 * i is written to position scatter_perm_q[bh][i] of o (and lse), i.e. the
 * inverse permutation is fused into the store; an entry outside [0, N) writes
 * nothing.
 * gather_perm_q (optional, int32 [B*Hq][N]): when set, q is unpermuted and
 * the query at permuted position i is row gather_perm_q[bh][i] of q (the
 * query gather fused into the load; an entry outside [0, N) reads zeros).
 * Neither permutation may be combined with causal (BSA_ERR_UNSUPPORTED).
 * scale <= 0 selects 1/sqrt(d).  A row with an empty list writes O = 0 and
 * LSE = -inf.  Log-weights must be finite or -inf.  crm (optional, device
 * uint32 [R][ceil(nQB/32)], the layout of bsa_crm_build): when set, each
 * row's list is the ascending walk of its CRM words (ScalingAttention,
 * section 7.3) and row_ptr/col are not read (may be NULL); it requires
 * v_layout = BSA_V_DIM_MAJOR and lw = NULL (else BSA_ERR_UNSUPPORTED).
 * Results are bit-identical to the CSR lists the same mask gives.
 * kv_share: 0, or 2 when query heads 2j and 2j + 1 of every KV-head group
 * have identical rows (same lists, same log-weights; grouped-query
 * attention whose block pattern is shared by the group's heads, e.g. the
 * Scatter/Gather prefill patterns of INTRA, section 4).  Then one launch
 * serves both rows of a pair, staging each K/V tile once for both heads; the
 * rows of head 2j + 1 are not read, and bsa_pair_rows_equal checks the
 * precondition.  Requires G = Hq / Hkv even, v_layout = BSA_V_DIM_MAJOR,
 * block = 128 and crm = NULL (else BSA_ERR_UNSUPPORTED); order then lists
 * rows of even heads only (bsa_schedule with head_step 2; other entries
 * compute nothing), n_order <= R / 2, and without order launch i serves the
 * i-th row of an even head.  Results equal those of kv_share = 0 on rows
 * that meet the precondition.
 * order2 (optional, int32 [n_order], with order): launch entry i also serves
 * row order2[i] when that is in [0, R), together with row order[i], staging
 * each K/V tile once for both.  Such a pair must list the same blocks in the
 * same order with the same log-weights (bit for bit) and lie in the same
 * batch and KV-head group (e.g. adjacent query blocks of one cluster of a
 * permuted head, which list identical blocks); bsa_schedule_pairs builds
 * such tables.  Entries with order2[i] outside [0, R) serve row order[i]
 * alone.  Requires kv_share = 0, v_layout = BSA_V_DIM_MAJOR, block = 128
 * and crm = NULL (else BSA_ERR_UNSUPPORTED); BSA_ERR_ARG without order.
 * Results equal those of the one-row launches within rounding (the pair
 * accumulates all of a row's keys in one softmax state, the single row in
 * two key halves merged at the end).
 * Asynchronous.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int32_t B, Hq, Hkv, d, block;
  int64_t N;
  int64_t q_str[3], k_str[3], v_str[3], o_str[3];
  const int32_t *row_ptr, *col;
  const float *lw;
  const int32_t *order;
  int64_t n_order; /* entries of order (launch count); 0 = R */
  const int32_t *scatter_perm_q;
  float scale;
  int32_t causal;
  int32_t v_layout; /* BSA_V_TOKEN_MAJOR or BSA_V_DIM_MAJOR */
  const uint32_t *crm; /* CRM rows in place of row_ptr/col, or NULL */
  const int32_t *gather_perm_q; /* query gather (int32 [B*Hq][N]), or NULL */
  int32_t kv_share; /* 0, or 2: rows of heads 2j and 2j + 1 of a KV group are identical */
  const int32_t *order2; /* second row of each launch entry (identical pair), or NULL */
} bsa_attn_args;

int bsa_attn_fwd(const bsa_attn_args *a, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Precondition check of bsa_attn_fwd's kv_share = 2: whether every pair of
 * query heads 2j, 2j + 1 within a KV-head group has identical rows, i.e.
 * for every b, even h and query block u the rows (b, h, u) and (b, h + 1, u)
 * list the same blocks in the same order with the same log-weights (bit
 * for bit; lw optional).  row_ptr: device int32 [B*Hq*nQB + 1]; col, lw:
 * device, as bsa_csr_fill writes them; equal: device int32 [1] (output, 1
 * if every pair is identical, else 0).  BSA_ERR_ARG for NULL pointers,
 * non-positive sizes, Hq % Hkv != 0; BSA_ERR_UNSUPPORTED when G = Hq / Hkv
 * is odd.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_pair_rows_equal(const int32_t *row_ptr, const int32_t *col, const float *lw, int32_t B, int32_t Hq,
                        int32_t Hkv, int32_t nQB, int32_t *equal, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Token-level attention over computational query sets.
 *
 * Source: INTRA, section 3 (a computational query set, CQS, is a group of
 * query tokens evaluated together, with structured mappings to the key
 * tokens it attends to) and section 4.8 (the selected Q, K and V tokens are
 * loaded and packed into dense on-chip tiles, outputs are scattered back to
 * the query positions, full or causal masking); MC-Sparse's token-level KV
 * selection per query group is the same computation.  For every query t of
 * set c: o_t = sum_e softmax_e(l_e) v_{s_e}, l_e = q_t . k_{s_e} * scale,
 * over the entries e of the set's key list (InstaGen, section 3.1
 * Eq. (1)-(3); one term per entry); entries outside [0, N) and, when causal,
 * keys s_e > t do not take part.  A query with no entry left gets O = 0 and
 * LSE = -inf.
 *
 * q [B][Hq][N][d], k and v [B][Hkv][N][d], o [B][Hq][N][d]: bf16 (uint16
 * bits) token-major device tensors addressed by the strides (d contiguous,
 * 16-byte aligned bases, strides multiples of 8; per-head byte extents
 * below 2^30); query head h reads KV head h / (Hq / Hkv).  n_sets sets per
 * head of set_size (64 or 128) query slots: q_idx (device int32
 * [B*Hq][n_sets][set_size]) holds each slot's query position, a position
 * outside [0, N) being an empty slot (nothing computed or written).  kv_ptr
 * (device int32 [B*Hq*n_sets + 1]) and kv_idx (device int32) list each set's
 * key positions, in any order.  o (and lse, float32 [B*Hq][N], optional) are
 * written at the query positions; a position should belong to at most one
 * set of its head (otherwise which write lands is unspecified).  o must not
 * alias q, k or v.  d must be 128 (BSA_ERR_UNSUPPORTED otherwise, and for
 * set_size outside {64, 128} or larger extents); BSA_ERR_ARG for NULL
 * pointers, non-positive sizes, Hq % Hkv != 0 or misaligned strides.
 * scale <= 0 selects 1/sqrt(d).  kv_share: 0, or s = 2 or 4 when every run
 * of s consecutive query heads s j .. s j + s - 1 of a KV-head group has
 * identical sets (same query slots, same key lists; INTRA's Scatter and
 * Gather maps hold for every head): then one workgroup serves the run's
 * sets, gathering each K/V tile once for all s heads; only the sets of head
 * s j are read.  Requires set_size = 64 and Hq / Hkv a multiple of s (else
 * BSA_ERR_UNSUPPORTED; other values BSA_ERR_ARG); results equal those of
 * kv_share = 0 on sets that meet the precondition, up to rounding order.
 * Asynchronous.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int32_t B, Hq, Hkv, d;
  int64_t N;
  int64_t q_str[3], k_str[3], v_str[3], o_str[3];
  int32_t n_sets, set_size;
  const int32_t *q_idx, *kv_ptr, *kv_idx;
  float scale;
  int32_t causal;
  int32_t kv_share; /* 0, or 2 or 4: runs of that many heads of a KV group have identical sets */
} bsa_tok_args;

int bsa_attn_tok_fwd(const bsa_tok_args *a, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Exact token-level KV selection, mass pass.
 *
 * Source: MC-Sparse, "The MC-Sparse Architecture" and Algorithm 1 (at an
 * anchor step, dense FlashAttention returns each query's log-sum-exp l_t;
 * exact KV selection then ranks, for every query group, the keys by the
 * attention probability mass the group's queries place on them).  For every
 * set c (a query group) and key s in [k0, k1):
 *   mass[c][s - k0] = sum over the set's queries t of exp(q_t . k_s * scale - l_t)
 * where l_t = lse[bh][t] (natural log, as bsa_attn_fwd writes it) and, when
 * causal, keys s > t add nothing for query t (lse must then come from a
 * causal pass).  Empty slots, and queries whose lse is -inf or NaN, add
 * nothing.
 *
 * q [B][Hq][N][d], k [B][Hkv][N][d]: bf16 (uint16 bits) token-major device
 * tensors addressed by the strides (d contiguous, 16-byte aligned bases,
 * strides multiples of 8; per-head byte extents below 2^30); query head h
 * reads KV head h / (Hq / Hkv).  lse: device float32 [B*Hq][N], contiguous.
 * q_idx: device int32 [B*Hq][n_sets][set_size] query positions, a position
 * outside [0, N) being an empty slot.  mass: device float32
 * [B*Hq*n_sets][k1 - k0], contiguous, fully written.  d must be 128 and
 * set_size 64 or 128 (BSA_ERR_UNSUPPORTED otherwise, and for larger
 * extents); BSA_ERR_ARG for NULL pointers, non-positive sizes, Hq % Hkv != 0,
 * misaligned strides or 0 <= k0 <= k1 <= N violated.  scale <= 0 selects
 * 1/sqrt(d).  The summation order is fixed: results are deterministic.
 * Asynchronous.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void *q, *k;
  const float *lse;
  float *mass;
  int32_t B, Hq, Hkv, d;
  int64_t N;
  int64_t q_str[3], k_str[3];
  int32_t n_sets, set_size;
  const int32_t *q_idx;
  int64_t k0, k1; /* key range of the output columns */
  float scale;
  int32_t causal;
} bsa_mass_args;

int bsa_group_mass(const bsa_mass_args *a, bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Exact token-level KV selection, top-K pass.
 *
 * Source: MC-Sparse, "The MC-Sparse Architecture" (each query group keeps the
 * K keys of largest attention mass: rank by score, take the top K, gather
 * their key and value vectors).  For each row r of x (device float32,
 * row stride ld >= n elements), idx[r][0 .. kk) (device int32, contiguous,
 * kk = min(k, n)) receives the column indices of the kk largest values in
 * ascending index order; among equal values the lower index is taken first
 * (-0 and +0 count as equal; NaN values must not occur).  kk = n lists every
 * column.  Nothing is enqueued for rows = 0 or k = 0.  BSA_ERR_ARG for NULL
 * pointers, n <= 0, ld < n, rows < 0 or k < 0; BSA_ERR_UNSUPPORTED for
 * n > 77824.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_topk_rows(const float *x, int64_t rows, int64_t n, int64_t ld, int32_t k, int32_t *idx,
                  bsa_stream_t stream);

/* ---------------------------------------------------------------------------
 * Engine-clock probe under MFMA load (for reading a measurement against the
 * clock the device sustains, not the path itself).  Launches `blocks`
 * workgroups of four wavefronts; each wavefront runs `iters` iterations of
 * four independent 32x32x16 bf16 MFMA chains (4 * iters * 32768 FLOP) and
 * writes, at ticks[2w] and ticks[2w + 1] (device uint64 [4 * blocks][2],
 * caller-owned), how far the shader clock counter and the 100 MHz real-time
 * counter advanced; the wavefront's clock is ticks[2w] / ticks[2w + 1] *
 * 100 MHz.  random_operands = 0: constant, low-entropy operands;
 * random_operands != 0: each lane cycles through eight A and eight B operands
 * of bf16 values drawn uniformly from [-2, 2), so every MFMA sees new random
 * bits (the clock under MFMA load falls as more operand bits switch).
 * BSA_ERR_ARG for NULL or non-positive sizes.  Asynchronous.
 * ------------------------------------------------------------------------- */
int bsa_clock_probe(int32_t blocks, int32_t iters, int32_t random_operands, uint64_t *ticks,
                    bsa_stream_t stream);

/* Number of compute units of the current device (for wave sizing), or a
 * negative error. */
int bsa_device_cus(void);

/* Peak engine clock of the current device in kHz (for reporting the clock a
 * measurement ran under), or a negative error. */
int bsa_device_clock_khz(void);

#ifdef __cplusplus
}
#endif
#endif /* BSATTN_H */
