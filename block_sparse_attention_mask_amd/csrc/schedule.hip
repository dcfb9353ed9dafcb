// Row schedule: the launch order of the attention kernel's workgroups.
//
// WaveAlign (section IV-D) cuts the row sequence into consecutive buckets of
// at most W rows (one wave of concurrently running rows) and sorts each bucket
// by descending nonzero-block count, so that long rows start first and short
// rows fill the tail next to the following wave; heads run one after another
// (section VI-B, sequential-head scheduling).  Here the row sequence is
// KV-group-major, so the query heads that share a KV head (GQA) run side by
// side on the same K/V blocks, and the order is a launch table read by the
// attention kernel: no data moves.
//
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  With n_xcd > 1 the sorted sequence is dealt so that XCD
// x receives the x-th contiguous slice, keeping neighbouring rows (which
// share K/V blocks) in one L2.
//
// A stage-1 order (WaveAlign section IV-C, bsa_spectral_order) may replace
// the query-block order within each head before the buckets are formed.
//
// With a head step of 2 only the first head of each pair of query heads that
// share a KV head is scheduled: the attention kernel that serves both heads'
// (identical) rows in one launch reads this table.
//
// One workgroup per bucket: keys (INT32_MAX - nnz) << 32 | position are
// sorted ascending with a bitonic network in LDS.
//
// With whole-segment buckets and the block lists given, a bucket keeps the
// sorted order only if consecutive rows share at least as many blocks as in
// the sequence order (the rows an XCD runs one after another reuse each
// other's K/V in its L2): sorting by length groups the rows of one cluster of
// a permuted head, but scatters the neighbouring rows of a banded or local
// pattern.  Shared blocks are estimated with a 256-bit signature per row (bit
// v mod 256 of each listed block v), kept in LDS.  When the sequence order
// wins, it is sorted longest-first within windows of kSeqWave consecutive
// rows (WaveAlign's intra-wave alignment, section IV-D, over a window of two
// XCD-waves of rows), which keeps neighbours together and balances each
// window.
//
// bsa_pair_rows_equal checks the precondition of that pair kernel: one
// wavefront per pair of rows compares lengths, block indices and log-weight
// bits, and clears a flag on any difference.
//
// bsa_schedule_pairs builds launch tables in which consecutive query blocks
// of a head with identical lists share one entry (the attention kernel then
// stages each K/V tile once for both rows).  Per bucket: each position
// compares its row with the same head's next one (lengths, signatures, then
// block indices and log-weight bits); one thread per head pairs greedily
// along its positions; the entries are keyed by tile count (2 nnz for a
// pair) and sorted as above, the adaptive choice taking each entry's first
// row; the second rows of pairs follow as empty entries.
#include "bsa_internal.h"

namespace {

constexpr int kMaxWave = 2048;
constexpr int kSeqWave = 64;   // rows per longest-first window of a sequence-order bucket

__device__ __forceinline__ int sig_fresh(const uint64_t *a, const uint64_t *prev) {
  int c = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) c += __popcll(a[w] & ~(prev ? prev[w] : 0ull));
  return c;
}

__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t *__restrict__ row_ptr,
                                                        const int32_t *__restrict__ col, int Hq, int Hkv,
                                                        int nQB, int W, int n_xcd, int64_t R,
                                                        const int32_t *__restrict__ row_perm, int hs,
                                                        int32_t *__restrict__ order) {
  __shared__ uint64_t key[kMaxWave];
  __shared__ uint64_t sig[kMaxWave][4];   // block signatures (adaptive mode)
  __shared__ int cost[2];                 // sorted, sequence
  const int G = Hq / Hkv, Gs = G / hs;   // scheduled heads per KV head: every hs-th
  const int64_t seg = (int64_t)Gs * nQB;
  const int64_t nbk = (seg + W - 1) / W;           // buckets per (b, g) segment
  const int64_t s = blockIdx.x / nbk, k = blockIdx.x % nbk;
  const int64_t start = s * seg + k * W;           // logical position of the bucket's first row
  const int n = (int)((k + 1) * W <= seg ? W : seg - k * W);
  int P2 = 1;
  while (P2 < n) P2 <<= 1;
  const int64_t b = s / Hkv, g = s % Hkv;
  // row at segment position j: head (b, g G + hs (j % Gs)), query block
  // j / Gs (or its stage-1 replacement); -1 for a corrupt stage-1 entry
  auto row_at = [&](int64_t j) -> int64_t {
    const int64_t p = j / Gs, h = b * Hq + g * G + hs * (j % Gs);
    const int64_t u = row_perm ? (int64_t)row_perm[h * nQB + p] : p;
    return (u >= 0 && u < nQB) ? h * nQB + u : -1;
  };
  for (int i = threadIdx.x; i < P2; i += 1024) {
    uint64_t kk = ~0ull;
    if (i < n) {
      const int64_t r = row_at(k * W + i);          // position within the segment
      const int32_t nnz = r >= 0 ? row_ptr[r + 1] - row_ptr[r] : 0;
      kk = ((uint64_t)(uint32_t)(0x7fffffff - nnz) << 32) | (uint32_t)i;
      if (col) {
        uint64_t sg[4] = {0, 0, 0, 0};
        auto add = [&](int32_t v) {
          const uint32_t bit = (uint32_t)v & 255u;
          sg[bit >> 6] |= 1ull << (bit & 63);
        };
        if (r >= 0) {
          const int32_t e1 = row_ptr[r + 1];
          int32_t e = row_ptr[r];
          // eight independent loads in flight per step
          for (; e + 8 <= e1; e += 8) {
            int32_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = col[e + j];
#pragma unroll
            for (int j = 0; j < 8; ++j) add(v[j]);
          }
          for (; e < e1; ++e) add(col[e]);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) sig[i][w] = sg[w];
      }
    }
    key[i] = kk;
  }
  if (threadIdx.x < 2) cost[threadIdx.x] = 0;
  __syncthreads();
  auto sort_keys = [&]() {
    for (int size = 2; size <= P2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = threadIdx.x; i < P2 / 2; i += 1024) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t a = key[lo], c = key[hi];
          if ((a > c) == up) {
            key[lo] = c;
            key[hi] = a;
          }
        }
        __syncthreads();
      }
    }
  };
  sort_keys();
  bool keep_seq = false;
  if (col) {
    int cs = 0, cq = 0;
    for (int i = threadIdx.x; i < n; i += 1024) {
      const int a = (int)(key[i] & 0xffffffffu), p = i ? (int)(key[i - 1] & 0xffffffffu) : 0;
      cs += sig_fresh(sig[a], i ? sig[p] : nullptr);
      cq += sig_fresh(sig[i], i ? sig[i - 1] : nullptr);
    }
    atomicAdd(&cost[0], cs);
    atomicAdd(&cost[1], cq);
    __syncthreads();
    keep_seq = cost[1] < cost[0];
    if (keep_seq) {
      // sequence order, longest-first within each window of kSeqWave rows:
      // keys (window, INT32_MAX - nnz, position) in 5 + 31 + 12 bits
      __syncthreads();
      for (int i = threadIdx.x; i < P2; i += 1024) {
        uint64_t kk = ~0ull;
        if (i < n) {
          const int64_t r = row_at(k * W + i);
          const int32_t nnz = r >= 0 ? row_ptr[r + 1] - row_ptr[r] : 0;
          kk = ((uint64_t)(i / kSeqWave) << 43) | ((uint64_t)(uint32_t)(0x7fffffff - nnz) << 12) | (uint32_t)i;
        }
        key[i] = kk;
      }
      __syncthreads();
      sort_keys();
    }
  }
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int src = (int)(key[i] & (keep_seq ? 0xfffu : 0xffffffffu));
    const int32_t r = (int32_t)row_at(k * W + src);
    const int64_t P = start + i;                    // logical position
    int64_t launch = P;
    if (n_xcd > 1) {
      int64_t st = 0;
      for (int x = 0; x < n_xcd; ++x) {
        const int64_t cnt = x < R ? (R - 1 - x) / n_xcd + 1 : 0;
        if (P < st + cnt) {
          launch = (P - st) * n_xcd + x;
          break;
        }
        st += cnt;
      }
    }
    order[launch] = r;
  }
}

// Paired launch tables (bsa_schedule_pairs): one workgroup per bucket of a
// (b, g) segment (head step 1, so G positions per query block, head inner).
__global__ __launch_bounds__(1024) void schedule_pairs_kernel(const int32_t *__restrict__ row_ptr,
                                                              const int32_t *__restrict__ col,
                                                              const float *__restrict__ lw, int Hq, int Hkv,
                                                              int nQB, int W, int adaptive, int n_xcd, int64_t R,
                                                              const int32_t *__restrict__ row_perm,
                                                              int32_t *__restrict__ order,
                                                              int32_t *__restrict__ order2) {
  __shared__ uint64_t key[kMaxWave];
  __shared__ uint64_t sig[kMaxWave][4];
  __shared__ int32_t rlen[kMaxWave];
  __shared__ int16_t upos[kMaxWave];       // entries in position order (adaptive cost)
  __shared__ int8_t same[kMaxWave], kind[kMaxWave];   // kind: 0 alone, 1 first of a pair, 2 second
  __shared__ int cost[2];
  __shared__ int n_units;
  const int G = Hq / Hkv;
  const int64_t seg = (int64_t)G * nQB;
  const int64_t nbk = (seg + W - 1) / W;
  const int64_t s = blockIdx.x / nbk, k = blockIdx.x % nbk;
  const int64_t start = s * seg + k * W;
  const int n = (int)((k + 1) * W <= seg ? W : seg - k * W);
  int P2 = 1;
  while (P2 < n) P2 <<= 1;
  const int64_t b = s / Hkv, g = s % Hkv;
  auto row_at = [&](int64_t j) -> int64_t {
    const int64_t p = j / G, h = b * Hq + g * G + j % G;
    const int64_t u = row_perm ? (int64_t)row_perm[h * nQB + p] : p;
    return (u >= 0 && u < nQB) ? h * nQB + u : -1;
  };
  // rows, lengths, signatures
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int64_t r = row_at(k * W + i);
    uint64_t sg[4] = {0, 0, 0, 0};
    int32_t len = 0;
    if (r >= 0) {
      const int32_t e1 = row_ptr[r + 1];
      int32_t e = row_ptr[r];
      len = e1 - e;
      auto add = [&](int32_t v) {
        const uint32_t bit = (uint32_t)v & 255u;
        sg[bit >> 6] |= 1ull << (bit & 63);
      };
      for (; e + 8 <= e1; e += 8) {
        int32_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = col[e + j];
#pragma unroll
        for (int j = 0; j < 8; ++j) add(v[j]);
      }
      for (; e < e1; ++e) add(col[e]);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) sig[i][w] = sg[w];
    rlen[i] = r >= 0 ? len : -1;
  }
  if (threadIdx.x < 2) cost[threadIdx.x] = 0;
  __syncthreads();
  // does position i list what the same head's next position lists?
  for (int i = threadIdx.x; i < n; i += 1024) {
    bool eq = false;
    const int c = i + G;
    if (c < n && rlen[i] >= 0 && rlen[i] == rlen[c] && sig[i][0] == sig[c][0] && sig[i][1] == sig[c][1] &&
        sig[i][2] == sig[c][2] && sig[i][3] == sig[c][3]) {
      const int64_t ra = row_at(k * W + i), rc = row_at(k * W + c);
      const int32_t a0 = row_ptr[ra], c0 = row_ptr[rc], len = rlen[i];
      eq = true;
      for (int32_t e = 0; eq && e < len; ++e) {
        eq = col[a0 + e] == col[c0 + e];
        if (lw) eq = eq && __float_as_uint(lw[a0 + e]) == __float_as_uint(lw[c0 + e]);
      }
    }
    same[i] = eq ? 1 : 0;
  }
  __syncthreads();
  // greedy pairing, one thread per head of the segment
  if (threadIdx.x < G) {
    bool second = false;
    for (int i = threadIdx.x; i < n; i += G) {
      int8_t kd = 0;
      if (second) {
        kd = 2;
        second = false;
      } else if (same[i]) {
        kd = 1;
        second = true;
      }
      kind[i] = kd;
    }
  }
  __syncthreads();
  auto cost_of = [&](int i) -> uint32_t {
    const int32_t len = rlen[i] > 0 ? rlen[i] : 0;
    return (uint32_t)(kind[i] == 1 ? 2 * len : len);
  };
  for (int i = threadIdx.x; i < P2; i += 1024) {
    uint64_t kk = ~0ull;
    if (i < n)
      kk = kind[i] == 2 ? ((1ull << 63) | (uint32_t)i)
                        : (((uint64_t)(0x7fffffffu - cost_of(i)) << 32) | (uint32_t)i);
    key[i] = kk;
  }
  __syncthreads();
  auto sort_keys = [&]() {
    for (int size = 2; size <= P2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int i = threadIdx.x; i < P2 / 2; i += 1024) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t a = key[lo], c = key[hi];
          if ((a > c) == up) {
            key[lo] = c;
            key[hi] = a;
          }
        }
        __syncthreads();
      }
    }
  };
  sort_keys();
  bool keep_seq = false;
  if (adaptive) {
    if (threadIdx.x == 0) {   // the entries in position order
      int m = 0;
      for (int i = 0; i < n; ++i)
        if (kind[i] != 2) upos[m++] = (int16_t)i;
      n_units = m;
    }
    __syncthreads();
    const int m = n_units;
    int cs = 0, cq = 0;
    for (int t = threadIdx.x; t < m; t += 1024) {
      const int a = (int)(key[t] & 0xffffffffu), pa = t ? (int)(key[t - 1] & 0xffffffffu) : 0;
      cs += sig_fresh(sig[a], t ? sig[pa] : nullptr);
      cq += sig_fresh(sig[upos[t]], t ? sig[upos[t - 1]] : nullptr);
    }
    atomicAdd(&cost[0], cs);
    atomicAdd(&cost[1], cq);
    __syncthreads();
    keep_seq = cost[1] < cost[0];
    if (keep_seq) {
      // position order, longest-first within windows of kSeqWave positions:
      // keys (window, INT32_MAX - cost, position) in 6 + 31 + 12 bits; the
      // second rows of pairs in window 63, after every entry
      __syncthreads();
      for (int i = threadIdx.x; i < P2; i += 1024) {
        uint64_t kk = ~0ull;
        if (i < n)
          kk = kind[i] == 2 ? ((63ull << 43) | (uint32_t)i)
                            : (((uint64_t)(i / kSeqWave) << 43) |
                               ((uint64_t)(0x7fffffffu - cost_of(i)) << 12) | (uint32_t)i);
        key[i] = kk;
      }
      __syncthreads();
      sort_keys();
    }
  }
  for (int i = threadIdx.x; i < n; i += 1024) {
    const int src = (int)(key[i] & (keep_seq ? 0xfffu : 0xffffffffu));
    int32_t r = -1, r2 = -1;
    if (kind[src] != 2) r = (int32_t)row_at(k * W + src);
    if (kind[src] == 1) r2 = (int32_t)row_at(k * W + src + G);
    const int64_t P = start + i;
    int64_t launch = P;
    if (n_xcd > 1) {
      int64_t st = 0;
      for (int x = 0; x < n_xcd; ++x) {
        const int64_t cnt = x < R ? (R - 1 - x) / n_xcd + 1 : 0;
        if (P < st + cnt) {
          launch = (P - st) * n_xcd + x;
          break;
        }
        st += cnt;
      }
    }
    order[launch] = r;
    order2[launch] = r2;
  }
}

__global__ void flag_set_kernel(int32_t *__restrict__ flag) {
  if (threadIdx.x == 0) flag[0] = 1;
}

__global__ __launch_bounds__(64) void pair_rows_equal_kernel(const int32_t *__restrict__ row_ptr,
                                                             const int32_t *__restrict__ col,
                                                             const float *__restrict__ lw, int nQB,
                                                             int32_t *__restrict__ equal) {
  const int64_t q = blockIdx.x, pr = q / nQB, u = q - pr * nQB;
  const int64_t r0 = 2 * pr * nQB + u, r1 = r0 + nQB;   // (b, 2j, u) and (b, 2j + 1, u)
  const int32_t a0 = row_ptr[r0], a1 = row_ptr[r0 + 1], b0 = row_ptr[r1], b1 = row_ptr[r1 + 1];
  bool diff = a1 - a0 != b1 - b0;
  if (!diff)
    for (int32_t i = threadIdx.x; i < a1 - a0; i += 64) {
      diff = diff || col[a0 + i] != col[b0 + i];
      if (lw) diff = diff || __float_as_uint(lw[a0 + i]) != __float_as_uint(lw[b0 + i]);
    }
  if (diff) equal[0] = 0;
}

}  // namespace

extern "C" int bsa_pair_rows_equal(const int32_t *row_ptr, const int32_t *col, const float *lw, int32_t B,
                                   int32_t Hq, int32_t Hkv, int32_t nQB, int32_t *equal, bsa_stream_t stream) {
  if (!row_ptr || !col || !equal || B <= 0 || Hq <= 0 || Hkv <= 0 || nQB <= 0) return BSA_ERR_ARG;
  if (Hq % Hkv) return BSA_ERR_ARG;
  if ((Hq / Hkv) % 2) return BSA_ERR_UNSUPPORTED;
  const int64_t pairs = (int64_t)B * (Hq / 2) * nQB;
  if (2 * pairs >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  hipStream_t s = bsa_hip_stream(stream);
  hipLaunchKernelGGL(flag_set_kernel, dim3(1), dim3(64), 0, s, equal);
  BSA_LAUNCH_CHECK();
  hipLaunchKernelGGL(pair_rows_equal_kernel, dim3((unsigned)pairs), dim3(64), 0, s, row_ptr, col, lw, nQB, equal);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_schedule(const int32_t *row_ptr, const int32_t *col, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t nQB, int32_t wave_rows, int32_t n_xcd, const int32_t *row_perm,
                            int32_t head_step, int32_t *order, bsa_stream_t stream) {
  if (!row_ptr || !order || B <= 0 || Hq <= 0 || Hkv <= 0 || nQB <= 0) return BSA_ERR_ARG;
  if (Hq % Hkv) return BSA_ERR_ARG;
  if (head_step != 1 && head_step != 2) return BSA_ERR_ARG;
  if ((Hq / Hkv) % head_step) return BSA_ERR_ARG;
  if (wave_rows < 0 || n_xcd < 0 || n_xcd > 64) return BSA_ERR_ARG;
  if (wave_rows > kMaxWave) return BSA_ERR_UNSUPPORTED;
  const int64_t R = (int64_t)B * Hq * nQB / head_step;   // rows scheduled
  if ((int64_t)B * Hq * nQB >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  // wave_rows = 0: one bucket per KV-group segment (up to 2048 rows), i.e. the
  // whole head longest-first, which measured fastest on MI355X together with
  // the XCD-contiguous deal
  const int W = wave_rows ? wave_rows : kMaxWave;
  const int64_t seg = (int64_t)(Hq / Hkv / head_step) * nQB;
  const int64_t grid = (int64_t)B * Hkv * ((seg + W - 1) / W);
  // the order choice applies to whole-segment buckets (wave_rows = 0)
  hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)grid), dim3(1024), 0, bsa_hip_stream(stream),
                     row_ptr, wave_rows ? nullptr : col, Hq, Hkv, nQB, W, n_xcd, R, row_perm, head_step, order);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_schedule_pairs(const int32_t *row_ptr, const int32_t *col, const float *lw, int32_t B,
                                  int32_t Hq, int32_t Hkv, int32_t nQB, int32_t wave_rows, int32_t n_xcd,
                                  const int32_t *row_perm, int32_t *order, int32_t *order2,
                                  bsa_stream_t stream) {
  if (!row_ptr || !col || !order || !order2 || B <= 0 || Hq <= 0 || Hkv <= 0 || nQB <= 0) return BSA_ERR_ARG;
  if (Hq % Hkv) return BSA_ERR_ARG;
  if (wave_rows < 0 || n_xcd < 0 || n_xcd > 64) return BSA_ERR_ARG;
  if (wave_rows > kMaxWave) return BSA_ERR_UNSUPPORTED;
  const int64_t R = (int64_t)B * Hq * nQB;
  if (R >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  const int W = wave_rows ? wave_rows : kMaxWave;
  if (Hq / Hkv > 1024) return BSA_ERR_UNSUPPORTED;   // one pairing thread per head of a segment
  const int64_t seg = (int64_t)(Hq / Hkv) * nQB;
  const int64_t grid = (int64_t)B * Hkv * ((seg + W - 1) / W);
  hipLaunchKernelGGL(schedule_pairs_kernel, dim3((unsigned)grid), dim3(1024), 0, bsa_hip_stream(stream), row_ptr,
                     col, lw, Hq, Hkv, nQB, W, wave_rows ? 0 : 1, n_xcd, R, row_perm, order, order2);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}
