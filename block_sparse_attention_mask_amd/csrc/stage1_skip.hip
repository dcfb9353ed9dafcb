// WaveAlign's adaptive skip of stage 1 (section IV-E, Runtime Coordination;
// section VI-F, Figure 13): the reordering is bypassed when its estimated
// latency reduction does not exceed its overhead.  The estimate is computed
// on the device from the CSR lists, so a pass that uses it makes no host
// round trip: the decision is a device flag that the stage-1 kernel reads.
//
// Statistics (integers, exact): nnz = listed entries (every entry is one
// tile the attention kernel processes), nmax = the largest per-head nnz,
// fresh = entries of each row whose block the previous row of the same head
// does not list (rows ascending, as the list builder writes them).  Then, in
// fp64: f = fresh / nnz, density = nnz / (BH nQB nKB), t_attn = nnz * tile_ms
// * (block/128)^2 * (d/128) / n_cus, gain = gamma f t_attn, cost = (iters/10)
// (row_ms nQB + nnz_ms nmax), K/V bytes of a head = 4 N d.  Stage 1 runs
// when the K/V of a head exceed l2_bytes, density >= density_min, gain > cost
// and the stage-1 kernel supports the shape.
//
// Three launches: the decision word is cleared; one wavefront per row looks
// every entry up in the previous row (binary search over the ascending list)
// and adds its fresh count to the decision word with an integer atomic; one
// workgroup reads nnz and nmax off the row offsets, forms the estimate and
// overwrites the word with the decision.  Integer sums do not depend on the
// order of the atomics, so the statistics and the decision do not depend on
// timing.
#include "bsa_internal.h"

// the decision's expressions are evaluated unfused, like the reference
// checker's, so both sides take it on the same fp64 values
#pragma clang fp contract(off)

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = kThreads / 64;   // one wavefront per row

__global__ void clear_kernel(int32_t *__restrict__ word) {
  if (threadIdx.x == 0) word[0] = 0;
}

__global__ __launch_bounds__(kThreads) void fresh_kernel(const int32_t *__restrict__ row_ptr,
                                                         const int32_t *__restrict__ col, int nQB, int64_t R,
                                                         int32_t *__restrict__ fresh) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const int u = (int)(r % nQB);
  const int32_t a0 = row_ptr[r], a1 = row_ptr[r + 1];
  const int32_t b0 = u > 0 ? row_ptr[r - 1] : a0, b1 = a0;   // the previous row (empty for u = 0)
  int32_t cnt = 0;
  for (int32_t e = a0 + lane; e < a1; e += 64) {
    const int32_t v = col[e];
    // first position in [b0, b1) holding a block >= v
    int32_t lo = b0, hi = b1;
    while (lo < hi) {
      const int32_t mid = lo + (hi - lo) / 2;
      if (col[mid] < v) lo = mid + 1;
      else hi = mid;
    }
    if (!(lo < b1 && col[lo] == v)) ++cnt;
  }
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if (lane == 0 && cnt) atomicAdd(fresh, cnt);
}

__global__ __launch_bounds__(kThreads) void stage1_decide_kernel(const int32_t *__restrict__ row_ptr, int BH,
                                                                 int nQB, int nKB, int64_t N, int d, int block,
                                                                 int iters, int n_cus, bsa_stage1_params prm,
                                                                 int32_t *__restrict__ decision,
                                                                 double *__restrict__ stats) {
  __shared__ int64_t red[kThreads];
  const int t = threadIdx.x;
  int64_t my_max = 0;
  for (int h = t; h < BH; h += kThreads) {
    const int64_t nh = (int64_t)row_ptr[(int64_t)(h + 1) * nQB] - row_ptr[(int64_t)h * nQB];
    if (nh > my_max) my_max = nh;
  }
  red[t] = my_max;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s && red[t + s] > red[t]) red[t] = red[t + s];
    __syncthreads();
  }
  if (t != 0) return;
  const int64_t nmax = red[0];
  const int64_t nnz = (int64_t)row_ptr[(int64_t)BH * nQB] - row_ptr[0];
  const int64_t fresh = decision[0];
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
  hipStream_t s = bsa_hip_stream(stream);
  const int64_t R = (int64_t)BH * nQB;
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(64), 0, s, decision);
  BSA_LAUNCH_CHECK();
  hipLaunchKernelGGL(fresh_kernel, dim3((unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(kThreads), 0, s,
                     row_ptr, col, nQB, R, decision);
  BSA_LAUNCH_CHECK();
  hipLaunchKernelGGL(stage1_decide_kernel, dim3(1), dim3(kThreads), 0, s, row_ptr, BH, nQB, nKB, N, d, block, iters,
                     n_cus, prm, decision, stats);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}
