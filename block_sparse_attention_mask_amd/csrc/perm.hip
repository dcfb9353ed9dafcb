// Cluster labels -> gather permutation, and row gather / scatter of bf16
// token-major tensors.
//
// Permuted block-sparse attention lays every cluster out contiguously before
// the block-sparse kernel (InstaGen, section 4) and restores the output order
// afterwards (WaveAlign, section V: permute query rows, restore outputs).
//
// perm_from_labels is a stable counting sort by (label, original index): one
// workgroup per (batch, head); each of its W wavefronts owns a contiguous
// W-th of the tokens (W = 16 for up to 1023 clusters, else 4).  Pass 1
// histograms labels per wavefront in LDS, a scan turns the histograms into
// per-(wavefront, label) write cursors in label-major order, pass 2 walks
// each wavefront's tokens in order 64 at a time: lanes with equal labels
// find each other with one ballot per label bit, take their rank among the
// lower lanes, and the lowest of them advances the cursor.  Both passes load
// eight 64-token groups of labels at once, so the loads overlap.
#include "bsa_internal.h"

namespace {

constexpr int kMaxClusters = 4095;  // + 1 overflow bucket for out-of-range labels
constexpr int kBatch = 8;           // 64-token groups of labels loaded at once

template <int W, int MAXB>
__global__ __launch_bounds__(64 * W) void perm_from_labels_kernel(const int32_t *__restrict__ labels, int64_t N,
                                                                  int C, int32_t *__restrict__ perm) {
  constexpr int NT = 64 * W;
  __shared__ int32_t cur[W][MAXB];
  __shared__ int32_t tot[NT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t bh = blockIdx.x;
  const int32_t *lab = labels + bh * N;
  int32_t *out = perm + bh * N;
  const int nb = C + 1;  // buckets; bucket C collects out-of-range labels
  for (int i = tid; i < W * nb; i += NT) cur[i / nb][i % nb] = 0;
  __syncthreads();
  const int64_t seg = (N + W - 1) / W;
  const int64_t s0 = wave * seg;
  const int64_t s1 = s0 + seg < N ? s0 + seg : N;
  auto bucket = [&](int32_t l) { return (l < 0 || l >= C) ? C : l; };
  for (int64_t t0 = s0; t0 < s1; t0 += 64 * kBatch) {
    int32_t l[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t t = t0 + 64 * k + lane;
      l[k] = t < s1 ? lab[t] : 0;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (t0 + 64 * k + lane < s1) atomicAdd(&cur[wave][bucket(l[k])], 1);
  }
  __syncthreads();
  // exclusive scan over entries e = bucket * W + wave (label-major)
  const int ne = nb * W;
  const int per = (ne + NT - 1) / NT;
  const int e0 = tid * per, e1 = e0 + per < ne ? e0 + per : ne;
  int32_t s = 0;
  for (int e = e0; e < e1; ++e) s += cur[e % W][e / W];
  tot[tid] = s;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int32_t x = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += x;
    __syncthreads();
  }
  int32_t run = tid ? tot[tid - 1] : 0;
  for (int e = e0; e < e1; ++e) {
    const int32_t x = cur[e % W][e / W];
    cur[e % W][e / W] = run;
    run += x;
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < nb) ++nbits;
  const uint64_t below = bsa_lanemask_lt(lane);
  for (int64_t t0 = s0; t0 < s1; t0 += 64 * kBatch) {
    int32_t l[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t t = t0 + 64 * k + lane;
      l[k] = t < s1 ? bucket(lab[t]) : 0;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int64_t c0 = t0 + 64 * k;
      if (c0 >= s1) break;
      const int64_t t = c0 + lane;
      const bool valid = t < s1;
      uint64_t same = __ballot(valid);
      for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (l[k] >> bit) & 1;
        const uint64_t bal = __ballot(set);
        same &= set ? bal : ~bal;
      }
      int32_t base = 0;
      if (valid) base = cur[wave][l[k]];
      __builtin_amdgcn_wave_barrier();
      if (valid) {
        const int rank = __popcll(same & below);
        out[base + rank] = (int32_t)t;
        if (rank == 0) cur[wave][l[k]] = base + __popcll(same);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// One thread moves 16 bytes (8 bf16); a row of d elements is d/8 threads.
template <bool kScatter>
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint16_t *__restrict__ src,
                                                           uint16_t *__restrict__ dst,
                                                           const int32_t *__restrict__ perm,
                                                           int H, int64_t N, int chunks,
                                                           int64_t ss0, int64_t ss1, int64_t ss2,
                                                           int64_t ds0, int64_t ds1, int64_t ds2,
                                                           int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int64_t row = gid / chunks;
  const int c = (int)(gid - row * chunks);
  const int64_t bh = row / N, i = row - bh * N;
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t j = perm[row];
  const bool ok = j >= 0 && j < N;
  if (kScatter) {
    if (!ok) return;
    const uint4 x = *reinterpret_cast<const uint4 *>(src + b * ss0 + h * ss1 + i * ss2 + c * 8);
    *reinterpret_cast<uint4 *>(dst + b * ds0 + h * ds1 + j * ds2 + c * 8) = x;
  } else {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (ok) x = *reinterpret_cast<const uint4 *>(src + b * ss0 + h * ss1 + j * ss2 + c * 8);
    *reinterpret_cast<uint4 *>(dst + b * ds0 + h * ds1 + i * ds2 + c * 8) = x;
  }
}

template <bool kScatter>
int permute_common(const void *src, void *dst, const int32_t *perm, int32_t B, int32_t H, int64_t N,
                   int32_t d, const int64_t ss[3], const int64_t ds[3], bsa_stream_t stream) {
  if (!src || !dst || !perm || !ss || !ds || B <= 0 || H <= 0 || N <= 0) return BSA_ERR_ARG;
  if (d != 64 && d != 128) return BSA_ERR_UNSUPPORTED;
  if (!bsa_aligned16(src) || !bsa_aligned16(dst)) return BSA_ERR_ARG;
  for (int i = 0; i < 3; ++i)
    if (ss[i] < 0 || ds[i] < 0 || (ss[i] & 7) || (ds[i] & 7)) return BSA_ERR_ARG;
  if (src == dst) return BSA_ERR_ARG;
  const int chunks = d / 8;
  const int64_t total = (int64_t)B * H * N * chunks;
  const int64_t grid = (total + 255) / 256;
  if (grid >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(permute_rows_kernel<kScatter>, dim3((unsigned)grid), dim3(256), 0,
                     bsa_hip_stream(stream), static_cast<const uint16_t *>(src),
                     static_cast<uint16_t *>(dst), perm, H, N, chunks, ss[0], ss[1], ss[2], ds[0],
                     ds[1], ds[2], total);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

// Gather + transpose: one thread turns an 8-token x 8-dim block into an
// 8-dim x 8-token block in registers (16-byte loads along d, 16-byte stores
// along tokens).  Threads are d-chunk fastest so that the gathered rows are
// read with full 256-byte segments.
__global__ __launch_bounds__(256) void transpose_rows_kernel(const uint16_t *__restrict__ src,
                                                             uint16_t *__restrict__ dst,
                                                             const int32_t *__restrict__ perm,
                                                             int H, int64_t N, int chunks, int64_t ld8,
                                                             int64_t ss0, int64_t ss1, int64_t ss2,
                                                             int64_t ds0, int64_t ds1, int64_t ds2,
                                                             int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int c = (int)(gid % chunks);                 // 8-dim chunk
  const int64_t rest = gid / chunks;
  const int64_t tg = rest % ld8;                     // 8-token group
  const int64_t bh = rest / ld8;
  const int64_t b = bh / H, h = bh - b * H;
  uint32_t w[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int64_t i = tg * 8 + t;
    int64_t j = -1;
    if (i < N) j = perm ? (int64_t)perm[bh * N + i] : i;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (j >= 0 && j < N) x = *reinterpret_cast<const uint4 *>(src + b * ss0 + h * ss1 + j * ss2 + c * 8);
    w[t][0] = x.x; w[t][1] = x.y; w[t][2] = x.z; w[t][3] = x.w;
  }
  uint16_t *out = dst + b * ds0 + h * ds1 + (int64_t)c * 8 * ds2 + tg * 8;
#pragma unroll
  for (int q = 0; q < 4; ++q) {   // dims 2q (low halves) and 2q+1 (high halves)
    const uint4 lo = make_uint4((w[0][q] & 0xffffu) | (w[1][q] << 16), (w[2][q] & 0xffffu) | (w[3][q] << 16),
                                (w[4][q] & 0xffffu) | (w[5][q] << 16), (w[6][q] & 0xffffu) | (w[7][q] << 16));
    const uint4 hi = make_uint4((w[0][q] >> 16) | (w[1][q] & 0xffff0000u), (w[2][q] >> 16) | (w[3][q] & 0xffff0000u),
                                (w[4][q] >> 16) | (w[5][q] & 0xffff0000u), (w[6][q] >> 16) | (w[7][q] & 0xffff0000u));
    *reinterpret_cast<uint4 *>(out + (2 * q) * ds2) = lo;
    *reinterpret_cast<uint4 *>(out + (2 * q + 1) * ds2) = hi;
  }
}

}  // namespace

extern "C" int bsa_transpose_rows(const void *src, void *dst, const int32_t *perm, int32_t B, int32_t H,
                                  int64_t N, int32_t d, int64_t ld, const int64_t ss[3],
                                  const int64_t ds[3], bsa_stream_t stream) {
  if (!src || !dst || !ss || !ds || B <= 0 || H <= 0 || N <= 0) return BSA_ERR_ARG;
  if (d != 64 && d != 128) return BSA_ERR_UNSUPPORTED;
  if (ld < N || (ld & 7) || ds[2] < ld) return BSA_ERR_ARG;
  if (!bsa_aligned16(src) || !bsa_aligned16(dst) || src == dst) return BSA_ERR_ARG;
  for (int i = 0; i < 3; ++i)
    if (ss[i] < 0 || ds[i] < 0 || (ss[i] & 7) || (ds[i] & 7)) return BSA_ERR_ARG;
  const int chunks = d / 8;
  const int64_t ld8 = ld / 8;
  const int64_t total = (int64_t)B * H * ld8 * chunks;
  const int64_t grid = (total + 255) / 256;
  if (grid >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(transpose_rows_kernel, dim3((unsigned)grid), dim3(256), 0, bsa_hip_stream(stream),
                     static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), perm, H, N, chunks,
                     ld8, ss[0], ss[1], ss[2], ds[0], ds[1], ds[2], total);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_perm_from_labels(const int32_t *labels, int64_t BH, int64_t N, int32_t n_clusters,
                                    int32_t *perm, bsa_stream_t stream) {
  if (!labels || !perm || BH < 0 || N < 0) return BSA_ERR_ARG;
  if (n_clusters <= 0) return BSA_ERR_ARG;
  if (n_clusters > kMaxClusters) return BSA_ERR_UNSUPPORTED;
  if (N >= (int64_t(1) << 31) || BH >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  if (BH == 0 || N == 0) return BSA_OK;
  if (n_clusters + 1 <= 1024)
    hipLaunchKernelGGL((perm_from_labels_kernel<16, 1024>), dim3((unsigned)BH), dim3(1024), 0,
                       bsa_hip_stream(stream), labels, N, n_clusters, perm);
  else
    hipLaunchKernelGGL((perm_from_labels_kernel<4, kMaxClusters + 1>), dim3((unsigned)BH), dim3(256), 0,
                       bsa_hip_stream(stream), labels, N, n_clusters, perm);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_permute_rows(const void *src, void *dst, const int32_t *perm, int32_t B, int32_t H,
                                int64_t N, int32_t d, const int64_t src_strides[3],
                                const int64_t dst_strides[3], bsa_stream_t stream) {
  return permute_common<false>(src, dst, perm, B, H, N, d, src_strides, dst_strides, stream);
}

extern "C" int bsa_unpermute_rows(const void *src, void *dst, const int32_t *perm, int32_t B,
                                  int32_t H, int64_t N, int32_t d, const int64_t src_strides[3],
                                  const int64_t dst_strides[3], bsa_stream_t stream) {
  return permute_common<true>(src, dst, perm, B, H, N, d, src_strides, dst_strides, stream);
}
