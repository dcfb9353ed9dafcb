// WaveAlign stage 1 (section IV-C): a polar spectral order of each head's
// query-block rows.
//
// A head's mask M (nQB rows x nKB KV blocks, 1 for listed blocks) is centred,
// C = M - 1 mu^T with mu the column means, which keeps pairwise row distances
// and sends the constant (workload) direction to a zero singular value
// (section IV-C.2).  The top-2 left singular subspace of C comes from
// subspace iteration X <- orth(C C^T X), applied without forming C:
// C^T X = M^T X - mu (1^T X), C Z = M Z - 1 (mu^T Z).  Rows are then ordered
// by the polar angle atan2(X[u][1], X[u][0]) of their rank-2 coordinates
// (section IV-C.1), ties by u.  The start X0[u] = (((37 u + 11) mod 101) /
// 101 - 1/2, ((53 u + 29) mod 97) / 97 - 1/2) and Gram-Schmidt for orth
// (a zero column stays zero).
//
// One workgroup per head, working in LDS.  The mask is held twice as a
// bitmask: column-major for M^T X (each column sums its rows in ascending
// order) and row-major for M Z (each row sums its blocks in ascending
// order); every sum over rows or columns is a fixed strided-then-tree
// reduction, so the result does not depend on timing.  Arithmetic is fp64
// (the work is O(nnz) per iteration).
#include <math.h>

#include "bsa_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxRows = 1024;             // nQB and nKB per head
constexpr int kMaxWords = 12288;           // words of each bitmask: nKB * ceil(nQB / 32), nQB * ceil(nKB / 32)

struct alignas(16) Sums {
  double a, b;
};

// Sum of (a, b) over the workgroup in a fixed order.
__device__ Sums block_sum2(double a, double b, double *red) {
  const int t = threadIdx.x;
  red[2 * t] = a;
  red[2 * t + 1] = b;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) {
      red[2 * t] += red[2 * (t + s)];
      red[2 * t + 1] += red[2 * (t + s) + 1];
    }
    __syncthreads();
  }
  const Sums r{red[0], red[1]};
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void spectral_order_kernel(const int32_t *__restrict__ row_ptr,
                                                                  const int32_t *__restrict__ col, int nQB,
                                                                  int nKB, int iters, int32_t *__restrict__ perm,
                                                                  double *__restrict__ angle,
                                                                  const int32_t *__restrict__ enable) {
  __shared__ uint32_t bits[kMaxWords];     // bits[v * nw + u / 32] bit u % 32: block v listed in row u
  __shared__ uint32_t rbits[kMaxWords];    // rbits[u * nwk + v / 32] bit v % 32: the same, row-major
  __shared__ double x1[kMaxRows], x2[kMaxRows], z1[kMaxRows], z2[kMaxRows], mu[kMaxRows];
  __shared__ double red[2 * kThreads];
  const int t = threadIdx.x;
  const int64_t bh = blockIdx.x;
  if (enable && enable[0] == 0) {   // the adaptive skip decided against stage 1: identity order
    for (int u = t; u < nQB; u += kThreads) {
      perm[bh * nQB + u] = u;
      if (angle) angle[bh * nQB + u] = 0.0;
    }
    return;
  }
  const int32_t *rp = row_ptr + bh * nQB;
  const int nw = (nQB + 31) / 32, nwk = (nKB + 31) / 32;

  for (int i = t; i < nKB * nw; i += kThreads) bits[i] = 0u;
  for (int i = t; i < nQB * nwk; i += kThreads) rbits[i] = 0u;
  __syncthreads();
  for (int u = t; u < nQB; u += kThreads)
    for (int32_t e = rp[u]; e < rp[u + 1]; ++e) {
      const int32_t v = col[e];
      if (v >= 0 && v < nKB) {
        atomicOr(&bits[v * nw + u / 32], 1u << (u % 32));
        atomicOr(&rbits[u * nwk + v / 32], 1u << (v % 32));
      }
    }
  __syncthreads();
  for (int v = t; v < nKB; v += kThreads) {
    int c = 0;
    for (int w = 0; w < nw; ++w) c += __popc(bits[v * nw + w]);
    mu[v] = (double)c / (double)nQB;
  }
  for (int u = t; u < nQB; u += kThreads) {
    x1[u] = (double)((37 * u + 11) % 101) / 101.0 - 0.5;
    x2[u] = (double)((53 * u + 29) % 97) / 97.0 - 0.5;
  }
  __syncthreads();

  for (int it = 0; it < iters; ++it) {
    // Z = C^T X
    double p1 = 0.0, p2 = 0.0;
    for (int u = t; u < nQB; u += kThreads) {
      p1 += x1[u];
      p2 += x2[u];
    }
    const Sums s = block_sum2(p1, p2, red);
    for (int v = t; v < nKB; v += kThreads) {
      double a1 = 0.0, a2 = 0.0;
      for (int w = 0; w < nw; ++w) {
        uint32_t m = bits[v * nw + w];
        while (m) {
          const int u = 32 * w + __builtin_ctz(m);
          m &= m - 1;
          a1 += x1[u];
          a2 += x2[u];
        }
      }
      z1[v] = a1 - mu[v] * s.a;
      z2[v] = a2 - mu[v] * s.b;
    }
    __syncthreads();
    // Y = C Z, into X (the sums of X are no longer needed)
    p1 = p2 = 0.0;
    for (int v = t; v < nKB; v += kThreads) {
      p1 += mu[v] * z1[v];
      p2 += mu[v] * z2[v];
    }
    const Sums tt = block_sum2(p1, p2, red);
    for (int u = t; u < nQB; u += kThreads) {
      double a1 = 0.0, a2 = 0.0;
      for (int w = 0; w < nwk; ++w) {
        uint32_t m = rbits[u * nwk + w];
        while (m) {
          const int v = 32 * w + __builtin_ctz(m);
          m &= m - 1;
          a1 += z1[v];
          a2 += z2[v];
        }
      }
      x1[u] = a1 - tt.a;
      x2[u] = a2 - tt.b;
    }
    __syncthreads();
    // Gram-Schmidt on the two columns
    p1 = 0.0;
    for (int u = t; u < nQB; u += kThreads) p1 += x1[u] * x1[u];
    const double n1 = sqrt(block_sum2(p1, 0.0, red).a);
    p2 = 0.0;
    for (int u = t; u < nQB; u += kThreads) {
      x1[u] = n1 > 0.0 ? x1[u] / n1 : 0.0;
      p2 += x1[u] * x2[u];
    }
    const double dd = block_sum2(p2, 0.0, red).a;
    p1 = 0.0;
    for (int u = t; u < nQB; u += kThreads) {
      x2[u] -= dd * x1[u];
      p1 += x2[u] * x2[u];
    }
    const double n2 = sqrt(block_sum2(p1, 0.0, red).a);
    for (int u = t; u < nQB; u += kThreads) x2[u] = n2 > 0.0 ? x2[u] / n2 : 0.0;
    __syncthreads();
  }

  // polar angle, then rank by (angle, u)
  for (int u = t; u < nQB; u += kThreads) {
    const double a = atan2(x2[u], x1[u]);
    z1[u] = a;
    if (angle) angle[bh * nQB + u] = a;
  }
  __syncthreads();
  for (int u = t; u < nQB; u += kThreads) {
    const double a = z1[u];
    int rank = 0;
    for (int j = 0; j < nQB; ++j) {
      const double b = z1[j];
      rank += (b < a) || (b == a && j < u);
    }
    perm[bh * nQB + rank] = u;
  }
}

}  // namespace

extern "C" int bsa_spectral_order(const int32_t *row_ptr, const int32_t *col, int32_t BH, int32_t nQB,
                                  int32_t nKB, int32_t iters, int32_t *perm, double *angle,
                                  const int32_t *enable, bsa_stream_t stream) {
  if (!row_ptr || !col || !perm || BH <= 0 || nQB <= 0 || nKB <= 0 || iters < 1) return BSA_ERR_ARG;
  if (nQB > kMaxRows || nKB > kMaxRows || (int64_t)nKB * ((nQB + 31) / 32) > kMaxWords ||
      (int64_t)nQB * ((nKB + 31) / 32) > kMaxWords)
    return BSA_ERR_UNSUPPORTED;
  if ((int64_t)BH * nQB >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(spectral_order_kernel, dim3((unsigned)BH), dim3(kThreads), 0, bsa_hip_stream(stream), row_ptr,
                     col, nQB, nKB, iters, perm, angle, enable);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}
