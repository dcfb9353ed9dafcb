// WaveAlign's adaptive skip of stage 1 (section IV-E, Runtime Coordination;
// section VI-F, Figure 13): the reordering is bypassed when its estimated
// latency reduction does not exceed its overhead.  The estimate is computed
// on the device from the CSR lists, so a pass that uses it makes no host
// round trip: the decision is a device flag that the stage-1 kernel reads.
//
// Statistics (integers, exact): nnz = listed blocks (entries in [0, nKB)),
// nmax = the largest per-head nnz, fresh = entries of each row that the
// previous row of the same head does not list (rows ascending, as the
// attention kernels require; a two-pointer merge per row).  Then, in fp64:
// f = fresh / nnz, density = nnz / (BH nQB nKB), t_attn = nnz * tile_ms *
// (block/128)^2 * (d/128) / n_cus, gain = gamma f t_attn, cost = (iters/10)
// (row_ms nQB + nnz_ms nmax), K/V bytes of a head = 4 N d.  Stage 1 runs when
// the K/V of a head exceed l2_bytes, density >= density_min, gain > cost and
// the stage-1 kernel supports the shape.
//
// One workgroup walks every head (its threads over the head's rows) and
// reduces in a fixed order, so the statistics and the decision do not depend
// on timing.
#include "bsa_internal.h"

// the decision's expressions are evaluated unfused, like the reference
// checker's, so both sides take it on the same fp64 values
#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 1024;

__device__ int64_t block_sum_i64(int64_t x, int64_t *red) {
  const int t = threadIdx.x;
  red[t] = x;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const int64_t r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void stage1_decide_kernel(const int32_t *__restrict__ row_ptr,
                                                                 const int32_t *__restrict__ col, int BH, int nQB,
                                                                 int nKB, int64_t N, int d, int block, int iters,
                                                                 int n_cus, bsa_stage1_params prm,
                                                                 int32_t *__restrict__ decision,
                                                                 double *__restrict__ stats) {
  __shared__ int64_t red[kThreads];
  const int t = threadIdx.x;
  int64_t nnz = 0, nmax = 0, fresh = 0;
  for (int h = 0; h < BH; ++h) {
    int64_t my_n = 0, my_f = 0;
    for (int u = t; u < nQB; u += kThreads) {
      const int64_t r = (int64_t)h * nQB + u;
      const int32_t a0 = row_ptr[r], a1 = row_ptr[r + 1];
      int32_t b = u > 0 ? row_ptr[r - 1] : a0;
      const int32_t b1 = a0;   // the previous row is [row_ptr[r - 1], a0), empty for u = 0
      for (int32_t e = a0; e < a1; ++e) {
        const int32_t v = col[e];
        if (v < 0 || v >= nKB) continue;
        ++my_n;
        // advance the previous row's pointer to the first entry >= v
        while (b < b1 && col[b] < v) ++b;
        if (!(b < b1 && col[b] == v)) ++my_f;
      }
    }
    const int64_t nh = block_sum_i64(my_n, red);
    const int64_t fh = block_sum_i64(my_f, red);
    nnz += nh;
    fresh += fh;
    if (nh > nmax) nmax = nh;
  }
  if (t != 0) return;
  const double f = nnz > 0 ? (double)fresh / (double)nnz : 0.0;
  const double density = (double)nnz / ((double)BH * (double)nQB * (double)nKB);
  const double bs = (double)block / 128.0;
  const double t_attn = (double)nnz * prm.tile_ms * bs * bs * ((double)d / 128.0) / (double)n_cus;
  const double gain = prm.gamma * f * t_attn;
  const double cost = ((double)iters / 10.0) * (prm.row_ms * (double)nQB + prm.nnz_ms * (double)nmax);
  const double footprint = 4.0 * (double)N * (double)d;
  const int64_t w1 = (nQB + 31) / 32, w2 = (nKB + 31) / 32;
  const int supported = nQB <= 1024 && nKB <= 1024 && nKB * w1 <= 12288 && nQB * w2 <= 12288;
  const int go = supported && footprint > prm.l2_bytes && density >= prm.density_min && gain > cost;
  decision[0] = go;
  if (stats) {
    stats[0] = f;
    stats[1] = density;
    stats[2] = t_attn;
    stats[3] = gain;
    stats[4] = cost;
    stats[5] = footprint;
    stats[6] = (double)go;
  }
}

}  // namespace

extern "C" void bsa_stage1_default_params(bsa_stage1_params *prm) {
  if (!prm) return;
  prm->gamma = 0.04;
  prm->tile_ms = 2.1e-3;
  prm->row_ms = 8.6e-4;
  prm->nnz_ms = 3.5e-6;
  prm->density_min = 0.10;
  prm->l2_bytes = 4.0 * 1024.0 * 1024.0;
}

extern "C" int bsa_stage1_decide(const int32_t *row_ptr, const int32_t *col, int32_t BH, int32_t nQB, int32_t nKB,
                                 int64_t N, int32_t d, int32_t block, int32_t iters, int32_t n_cus,
                                 const bsa_stage1_params *params, int32_t *decision, double *stats,
                                 bsa_stream_t stream) {
  if (!row_ptr || !col || !decision || BH <= 0 || nQB <= 0 || nKB <= 0 || N <= 0 || d <= 0 || block <= 0 ||
      iters < 1 || n_cus <= 0)
    return BSA_ERR_ARG;
  if ((int64_t)BH * nQB >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  bsa_stage1_params prm;
  if (params) prm = *params;
  else bsa_stage1_default_params(&prm);
  hipLaunchKernelGGL(stage1_decide_kernel, dim3(1), dim3(kThreads), 0, bsa_hip_stream(stream), row_ptr, col, BH,
                     nQB, nKB, N, d, block, iters, n_cus, prm, decision, stats);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}
