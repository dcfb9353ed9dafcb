// Block mask / threshold map -> CSR lists of KV blocks per query-block row.
//
// Keep rule (ScalingAttention, section 5.2, Eq. 2: M_p = I(T <= p)): entry
// (r, v) is kept when mask != 0, or T <= p, or it is the forced diagonal.
// Rows come out in ascending KV-block order, the order in which the CRM
// iterator (ScalingAttention, section 7.3, Algorithm 2) walks active blocks.
//
// CRM rows (section 7.2) come from the same keep rule: each 64-block ballot
// is two words of the row.  The row counts of CRM rows (popcounts) feed the
// same scan, and the CRM -> CSR conversion walks each row's bits in
// ascending order.
//
// Pass 1 counts each row with one wavefront (ballot + popcount over 64 KV
// blocks per step), a single-workgroup scan turns counts into row_ptr, pass 2
// writes each row's ascending list with the same ballot, placing lane i at
// the popcount of the keep bits below it.  All integer work: deterministic.
#include "bsa_internal.h"

namespace {

constexpr int kRowsPerBlock = 4;  // one wavefront per row, 256 threads

__device__ __forceinline__ bool keep_entry(const uint8_t *mask, const float *T, float p, int64_t idx) {
  return mask ? (mask[idx] != 0) : (T[idx] <= p);
}

__global__ __launch_bounds__(256) void csr_count_kernel(const uint8_t *__restrict__ mask,
                                                        const float *__restrict__ T, float p,
                                                        int64_t R, int nQB, int nKB, int force_diag,
                                                        int32_t *__restrict__ row_ptr) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const int u = (int)(r % nQB);
  const int64_t base = r * nKB;
  int cnt = 0;
  for (int v0 = 0; v0 < nKB; v0 += 64) {
    const int v = v0 + lane;
    bool k = false;
    if (v < nKB) k = keep_entry(mask, T, p, base + v) || (force_diag && v == u);
    cnt += __popcll(__ballot(k));
  }
  if (lane == 0) row_ptr[r + 1] = cnt;
}

// In-place inclusive scan of row_ptr[1..R] (counts) with row_ptr[0] = 0.
__global__ __launch_bounds__(1024) void csr_scan_kernel(int32_t *__restrict__ row_ptr, int64_t R) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (R + 1023) / 1024;
  const int64_t beg = 1 + (int64_t)t * per;
  const int64_t end = beg + per < R + 1 ? beg + per : R + 1;
  int32_t s = 0;
  for (int64_t i = beg; i < end; ++i) s += row_ptr[i];
  part[t] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 partial sums
  for (int off = 1; off < 1024; off <<= 1) {
    int32_t x = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  int32_t run = t ? part[t - 1] : 0;
  for (int64_t i = beg; i < end; ++i) {
    run += row_ptr[i];
    row_ptr[i] = run;
  }
  if (t == 0) row_ptr[0] = 0;
}

__global__ __launch_bounds__(256) void csr_fill_kernel(const uint8_t *__restrict__ mask,
                                                       const float *__restrict__ T, float p,
                                                       const uint32_t *__restrict__ lw_map_bits,
                                                       int64_t R, int nQB, int nKB, int force_diag,
                                                       const int32_t *__restrict__ row_ptr,
                                                       int32_t *__restrict__ col,
                                                       uint32_t *__restrict__ lw_bits,
                                                       int64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const int u = (int)(r % nQB);
  const int64_t base = r * nKB;
  int64_t out = row_ptr[r];
  const uint64_t below = bsa_lanemask_lt(lane);
  for (int v0 = 0; v0 < nKB; v0 += 64) {
    const int v = v0 + lane;
    bool k = false;
    if (v < nKB) k = keep_entry(mask, T, p, base + v) || (force_diag && v == u);
    const uint64_t bal = __ballot(k);
    if (k) {
      const int64_t e = out + __popcll(bal & below);
      if (e >= 0 && e < capacity) {
        col[e] = v;
        if (lw_bits) lw_bits[e] = lw_map_bits ? lw_map_bits[base + v] : 0u;
      }
    }
    out += __popcll(bal);
  }
}

// CRM rows: one wavefront per row; each ballot over 64 KV blocks is two
// words of the row, written by lanes 0 and 1.
__global__ __launch_bounds__(256) void crm_build_kernel(const uint8_t *__restrict__ mask,
                                                        const float *__restrict__ T, float p, int64_t R,
                                                        int nQB, int nKB, int force_diag,
                                                        uint32_t *__restrict__ crm) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const int u = (int)(r % nQB);
  const int64_t base = r * nKB;
  const int W = bsa_crm_words(nKB);
  uint32_t *row = crm + r * W;
  for (int v0 = 0; v0 < nKB; v0 += 64) {
    const int v = v0 + lane;
    bool k = false;
    if (v < nKB) k = keep_entry(mask, T, p, base + v) || (force_diag && v == u);
    const uint64_t bal = __ballot(k);
    const int w = v0 / 32 + lane;
    if (lane < 2 && w < W) row[w] = (uint32_t)(bal >> (32 * lane));
  }
}

// Per-row block counts of CRM rows into row_ptr[r + 1].
__global__ __launch_bounds__(256) void crm_count_kernel(const uint32_t *__restrict__ crm, int64_t R, int nKB,
                                                        int32_t *__restrict__ row_ptr) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const int W = bsa_crm_words(nKB);
  const int c = bsa_crm_count(crm + r * W, W, bsa_crm_tail(nKB), lane);
  if (lane == 0) row_ptr[r + 1] = c;
}

// CRM rows -> ascending CSR lists by the forward walk.
__global__ __launch_bounds__(256) void crm_to_csr_kernel(const uint32_t *__restrict__ crm, int64_t R, int nKB,
                                                         const int32_t *__restrict__ row_ptr,
                                                         int32_t *__restrict__ col, int64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= R) return;
  const int W = bsa_crm_words(nKB);
  const int64_t e0 = row_ptr[r], n = (int64_t)row_ptr[r + 1] - e0;
  const int64_t room = capacity - e0;
  const int lim = (int)(n < room ? n : room);
  if (e0 < 0 || lim <= 0) return;
  bsa_crm_walk(crm + r * W, W, bsa_crm_tail(nKB), 0, lim, col + e0, 0, 1, lane);
}

int check_csr_args(const uint8_t *mask, const float *T, int64_t R, int32_t nQB, int32_t nKB,
                   int force_diag, const void *row_ptr) {
  if (!row_ptr || R < 0 || nQB <= 0 || nKB <= 0) return BSA_ERR_ARG;
  if ((mask == nullptr) == (T == nullptr)) return BSA_ERR_ARG;
  if (R > 0 && R * (int64_t)nKB >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  if (force_diag && nQB > nKB) return BSA_ERR_UNSUPPORTED;
  return BSA_OK;
}

}  // namespace

extern "C" int bsa_csr_count(const uint8_t *mask, const float *T, float p, int64_t R, int32_t nQB,
                             int32_t nKB, int force_diag, int32_t *row_ptr, int64_t *nnz_out,
                             bsa_stream_t stream) {
  int rc = check_csr_args(mask, T, R, nQB, nKB, force_diag, row_ptr);
  if (rc) return rc;
  hipStream_t s = bsa_hip_stream(stream);
  if (R > 0) {
    const unsigned grid = (unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock);
    hipLaunchKernelGGL(csr_count_kernel, dim3(grid), dim3(256), 0, s, mask, T, p, R, nQB, nKB,
                       force_diag, row_ptr);
    BSA_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, row_ptr, R);
  BSA_LAUNCH_CHECK();
  if (nnz_out) {
    int32_t n = 0;
    BSA_HIP(hipMemcpyAsync(&n, row_ptr + R, sizeof(n), hipMemcpyDeviceToHost, s));
    BSA_HIP(hipStreamSynchronize(s));
    *nnz_out = n;
  }
  return BSA_OK;
}

extern "C" int bsa_csr_fill(const uint8_t *mask, const float *T, float p, const float *lw_map,
                            int64_t R, int32_t nQB, int32_t nKB, int force_diag,
                            const int32_t *row_ptr, int32_t *col, float *lw, int64_t capacity,
                            bsa_stream_t stream) {
  int rc = check_csr_args(mask, T, R, nQB, nKB, force_diag, row_ptr);
  if (rc) return rc;
  if (capacity < 0) return BSA_ERR_ARG;
  if (!col && capacity > 0) return BSA_ERR_ARG;
  if (R == 0) return BSA_OK;
  const unsigned grid = (unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(csr_fill_kernel, dim3(grid), dim3(256), 0, bsa_hip_stream(stream), mask, T, p,
                     reinterpret_cast<const uint32_t *>(lw_map), R, nQB, nKB, force_diag, row_ptr,
                     col, reinterpret_cast<uint32_t *>(lw), capacity);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_crm_build(const uint8_t *mask, const float *T, float p, int64_t R, int32_t nQB,
                             int32_t nKB, int force_diag, uint32_t *crm, bsa_stream_t stream) {
  int rc = check_csr_args(mask, T, R, nQB, nKB, force_diag, crm);
  if (rc) return rc;
  if (R == 0) return BSA_OK;
  const unsigned grid = (unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(crm_build_kernel, dim3(grid), dim3(256), 0, bsa_hip_stream(stream), mask, T, p, R, nQB,
                     nKB, force_diag, crm);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_crm_row_ptr(const uint32_t *crm, int64_t R, int32_t nKB, int32_t *row_ptr, int64_t *nnz_out,
                               bsa_stream_t stream) {
  if (!row_ptr || R < 0 || nKB <= 0 || (R > 0 && !crm)) return BSA_ERR_ARG;
  if (R > 0 && R * (int64_t)nKB >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  hipStream_t s = bsa_hip_stream(stream);
  if (R > 0) {
    const unsigned grid = (unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock);
    hipLaunchKernelGGL(crm_count_kernel, dim3(grid), dim3(256), 0, s, crm, R, nKB, row_ptr);
    BSA_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(1024), 0, s, row_ptr, R);
  BSA_LAUNCH_CHECK();
  if (nnz_out) {
    int32_t n = 0;
    BSA_HIP(hipMemcpyAsync(&n, row_ptr + R, sizeof(n), hipMemcpyDeviceToHost, s));
    BSA_HIP(hipStreamSynchronize(s));
    *nnz_out = n;
  }
  return BSA_OK;
}

extern "C" int bsa_crm_to_csr(const uint32_t *crm, int64_t R, int32_t nKB, const int32_t *row_ptr, int32_t *col,
                              int64_t capacity, bsa_stream_t stream) {
  if (!row_ptr || R < 0 || nKB <= 0 || capacity < 0 || (R > 0 && !crm)) return BSA_ERR_ARG;
  if (!col && capacity > 0) return BSA_ERR_ARG;
  if (R > 0 && R * (int64_t)nKB >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  if (R == 0 || capacity == 0) return BSA_OK;
  const unsigned grid = (unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL(crm_to_csr_kernel, dim3(grid), dim3(256), 0, bsa_hip_stream(stream), crm, R, nKB, row_ptr,
                     col, capacity);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_version(void) { return (0 << 16) | 1; }

extern "C" const char *bsa_strerror(int code) {
  switch (code) {
    case BSA_OK: return "ok";
    case BSA_ERR_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case BSA_ERR_HIP: return "HIP runtime or launch failure";
    default: return "unknown error";
  }
}

extern "C" int bsa_device_cus(void) {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return BSA_ERR_HIP;
  return n;
}

extern "C" int bsa_device_clock_khz(void) {
  int dev = 0, k = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BSA_ERR_HIP;
  if (hipDeviceGetAttribute(&k, hipDeviceAttributeClockRate, dev) != hipSuccess) return BSA_ERR_HIP;
  return k;
}
