// Group-shared importance sampling over KV tiles (InstaGen, Algorithm 1
// steps 2-13; section 3.2.1 Eq. 4; the systematic PPS sample of section 4),
// and the centroids it scores.
//
// Centroids: the tokens of one label are one contiguous segment of the
// label-sorted sequence (bsa_segment_offsets), and a centroid is the mean of
// its segment's rows (bsa_segment_means); fixed-length segments give the
// mean key of every KV tile.
//
// Sampler: one workgroup per (head, query group).  The tile is the unit of
// Algorithm 1 at tile granularity: its centroid is its mean key and its
// size its number of real keys.  The workgroup computes the tile masses
// |v| exp(scale q_g . k_v - max) in fp64, finds the m_exact + m_sample
// largest in (mass descending, tile ascending) order (the only ranks the
// rest needs), takes the m_exact largest as the exact set, water-fills the
// inclusion probabilities of the rest (Eq. 4: the number k of capped tiles
// is the smallest k for which the k-th largest residual mass is not capped
// by lam = (m - k) / (sum of the masses from the k-th on)), draws the
// systematic PPS sample (points u0 + j of the running sum of pi over the
// residual in ascending tile order), and writes the mask and log-weight rows
// (-ln pi for a sampled tile with pi < 1, else 0; 0 on the diagonal) of every
// query block of the group.  Sums over tiles are fixed-order reductions and
// scans, so the result does not depend on timing.
#include <math.h>

#include "bsa_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxTiles = 1024;   // KV tiles per head
constexpr int kMaxD = 256;
constexpr int kPer = kMaxTiles / kThreads;

// ---------------------------------------------------------------- offsets
constexpr int kOffThreads = 1024;
constexpr int kMaxGroups = 8192;

__global__ __launch_bounds__(kOffThreads) void segment_offsets_kernel(const int32_t *__restrict__ labels, int64_t N,
                                                                      int G, int32_t *__restrict__ seg_ptr) {
  __shared__ int32_t cnt[kMaxGroups + 1];
  __shared__ int32_t part[kOffThreads];
  const int t = threadIdx.x;
  const int64_t bh = blockIdx.x;
  for (int g = t; g <= G; g += kOffThreads) cnt[g] = 0;
  __syncthreads();
  const int32_t *lab = labels + bh * N;
  for (int64_t i = t; i < N; i += kOffThreads) {
    const int32_t l = lab[i];
    if (l >= 0 && l < G) atomicAdd(&cnt[l + 1], 1);
  }
  __syncthreads();
  // exclusive offsets: each thread scans a contiguous run of counts, then the
  // run totals are scanned
  const int per = (G + 1 + kOffThreads - 1) / kOffThreads;
  const int lo = t * per, hi = lo + per < G + 1 ? lo + per : G + 1;
  int32_t s = 0;
  for (int g = lo; g < hi; ++g) s += cnt[g];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < kOffThreads; off <<= 1) {
    const int32_t x = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += x;
    __syncthreads();
  }
  int32_t run = t ? part[t - 1] : 0;
  int32_t *sp = seg_ptr + bh * (G + 1);
  for (int g = lo; g < hi; ++g) {
    run += cnt[g];
    sp[g] = run;
  }
}

// ------------------------------------------------------------------ means
// Thread (row phase rp, column group cg) sums 8 columns of rows
// lo + rp, lo + rp + NP, ... in fp32; the NP partial sums of a column are
// then added in row-phase order.
__global__ __launch_bounds__(kThreads) void segment_means_kernel(const uint16_t *__restrict__ x, int64_t xs0,
                                                                 int64_t xs1, int64_t xs2, int H, int64_t N, int d,
                                                                 const int32_t *__restrict__ seg_ptr, int G,
                                                                 int seg_len, float *__restrict__ means) {
  __shared__ float red[kThreads * 8];
  const int t = threadIdx.x;
  const int s = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / H, h = bh % H;
  int64_t lo, hi;
  if (seg_ptr) {
    lo = seg_ptr[bh * (G + 1) + s];
    hi = seg_ptr[bh * (G + 1) + s + 1];
  } else {
    lo = (int64_t)s * seg_len;
    hi = lo + seg_len < N ? lo + seg_len : N;
  }
  if (lo < 0) lo = 0;
  if (hi > N) hi = N;
  const int ncg = d / 8, np = kThreads / ncg;
  const int cg = t % ncg, rp = t / ncg;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (rp < np) {
    const uint16_t *base = x + b * xs0 + h * xs1 + cg * 8;
    for (int64_t i = lo + rp; i < hi; i += np) {
      const uint4 w = *reinterpret_cast<const uint4 *>(base + i * xs2);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(u[j] << 16);
        acc[2 * j + 1] += __uint_as_float(u[j] & 0xffff0000u);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[t * 8 + j] = acc[j];
  __syncthreads();
  const int64_t n = hi - lo;
  float *out = means + (bh * G + s) * d;
  for (int c = t; c < d; c += kThreads) {
    const int g8 = c / 8, j = c % 8;
    float sum = 0.f;
    for (int r = 0; r < np; ++r) sum += red[(r * ncg + g8) * 8 + j];
    out[c] = n > 0 ? sum / (float)n : 0.f;
  }
}

// ---------------------------------------------------------------- sampler
__device__ double block_max(double v, double *red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] = fmax(red[t], red[t + s]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ double block_sum(double v, double *red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// In-place inclusive scan of a[0..n) (n <= kMaxTiles): each thread scans its
// kPer consecutive entries, the thread totals are scanned (Hillis-Steele),
// and each thread adds the total before it.
__device__ void block_scan(double *a, int n, double *tot) {
  const int t = threadIdx.x;
  const int lo = t * kPer;
  double s = 0.0;
  for (int i = lo; i < lo + kPer && i < n; ++i) {
    s += a[i];
    a[i] = s;
  }
  tot[t] = s;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const double x = t >= off ? tot[t - off] : 0.0;
    __syncthreads();
    tot[t] += x;
    __syncthreads();
  }
  const double before = t ? tot[t - 1] : 0.0;
  for (int i = lo; i < lo + kPer && i < n; ++i) a[i] += before;
  __syncthreads();
}

// Ranks up to this many are found by rounds of a workgroup-wide argmax;
// larger selections count, for every tile, the tiles before it.
constexpr int kTopFast = 64;

__global__ __launch_bounds__(kThreads) void is_sample_kernel(
    const float *__restrict__ qbar, const float *__restrict__ kbar, const int32_t *__restrict__ q_seg_ptr,
    const double *__restrict__ uoff, int Hq, int Hkv, int G, int64_t N, int block, int d, int m_exact,
    int m_sample, double scale, uint8_t *__restrict__ mask, float *__restrict__ lw_map,
    double *__restrict__ pi_out) {
  // per tile: its mass; the running sum of pi in tile order (before that, the
  // residual's suffix sums); its rank in (mass descending, tile ascending)
  // order where that is below K, else K
  __shared__ double mass[kMaxTiles], cum[kMaxTiles];
  __shared__ int32_t rk[kMaxTiles];
  __shared__ int32_t top[kMaxTiles];   // top[j]: the tile of rank j, j < K
  __shared__ float lwv[kMaxTiles];
  __shared__ uint8_t keep[kMaxTiles];
  __shared__ float qs[kMaxD];
  __shared__ double red[kThreads];
  __shared__ double lam_s;
  __shared__ int k_s;
  const int t = threadIdx.x;
  const int g = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t b = bh / Hq, h = bh % Hq;
  const int64_t gk = b * Hkv + h / (Hq / Hkv);
  const int nb = (int)((N + block - 1) / block);
  const int32_t *sp = q_seg_ptr + bh * (G + 1);
  const int64_t s0 = sp[g], s1 = sp[g + 1];
  int u0 = (int)((s0 + block - 1) / block), u1 = (int)((s1 + block - 1) / block);
  if (u1 > nb) u1 = nb;
  if (u0 < 0) u0 = 0;
  if (g == G - 1) {   // rows after the last labelled token belong to no group
    for (int64_t r = bh * nb + u1; r < (bh + 1) * nb; ++r)
      for (int v = t; v < nb; v += kThreads) {
        mask[r * nb + v] = 0;
        lw_map[r * nb + v] = 0.f;
      }
  }
  if (pi_out)
    for (int v = t; v < nb; v += kThreads) pi_out[(bh * G + g) * nb + v] = 0.0;
  if (u0 >= u1) return;

  // step 2: centroid scores and tile masses.  A thread's tiles are
  // v = t + kThreads i; their dot products run as independent chains (each
  // in order over the dims), tiles past the last reading the last one's row.
  for (int c = t; c < d; c += kThreads) qs[c] = qbar[(bh * G + g) * d + c];
  __syncthreads();
  constexpr int kPerT = kMaxTiles / kThreads;
  double dot[kPerT];
  const float *kv[kPerT];
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    const int v = t + kThreads * i;
    kv[i] = kbar + (gk * nb + (v < nb ? v : nb - 1)) * d;
    dot[i] = 0.0;
  }
  for (int c = 0; c < d; ++c) {
    const double qc = (double)qs[c];
#pragma unroll
    for (int i = 0; i < kPerT; ++i) dot[i] += qc * (double)kv[i][c];
  }
  double amax = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPerT; ++i) {
    const int v = t + kThreads * i;
    if (v < nb) {
      mass[v] = scale * dot[i];
      amax = fmax(amax, mass[v]);
    }
  }
  amax = block_max(amax, red);
  const int ne = m_exact < nb ? m_exact : nb;
  const int nr = nb - ne;
  const bool capped = nr > m_sample;              // the residual needs water-filling
  const int K = capped ? ne + m_sample : ne;      // ranks needed: the exact set and the residual's largest
  for (int v = t; v < nb; v += kThreads) {
    const int64_t size = N - (int64_t)v * block < block ? N - (int64_t)v * block : block;
    mass[v] = (double)size * exp(mass[v] - amax);
    rk[v] = K;
  }
  for (int j = t; j < K; j += kThreads) top[j] = 0;
  __syncthreads();

  // step 4: the K first tiles in (mass descending, tile ascending) order;
  // the exact set is the first m_exact.  For K <= kTopFast every wavefront
  // takes its own K first tiles by K rounds of a wavefront argmax over its
  // lanes' tiles (registers and shuffles only); every tile among the K first
  // overall is among its wavefront's K first, so counting within the union
  // of the wavefronts' lists gives those tiles their rank, and every other
  // candidate a count of at least K.
  if (K <= kTopFast) {
    double* const cm = cum;                                  // candidates' masses (cum is free here)
    int32_t* const cv = reinterpret_cast<int32_t *>(lwv);   // and tiles (lwv is free here)
    const int lane = t & 63, wave = t >> 6;
    double m[kPerT];
    bool avail[kPerT];
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int v = t + kThreads * i;
      avail[i] = v < nb;
      m[i] = avail[i] ? mass[v] : 0.0;
    }
    for (int j = 0; j < K; ++j) {
      double bm = -1.0;   // masses are >= 0
      int bv = nb;
#pragma unroll
      for (int i = 0; i < kPerT; ++i) {
        const int v = t + kThreads * i;
        if (avail[i] && (m[i] > bm || (m[i] == bm && v < bv))) {
          bm = m[i];
          bv = v;
        }
      }
      for (int off = 32; off > 0; off >>= 1) {
        const double om = __shfl_xor(bm, off);
        const int ov = __shfl_xor(bv, off);
        if (om > bm || (om == bm && ov < bv)) {
          bm = om;
          bv = ov;
        }
      }
#pragma unroll
      for (int i = 0; i < kPerT; ++i)
        if (t + kThreads * i == bv) avail[i] = false;
      if (lane == 0) {
        cm[wave * K + j] = bm;
        cv[wave * K + j] = bv;
      }
    }
    __syncthreads();
    const int nc = (kThreads / 64) * K;
    for (int c = t; c < nc; c += kThreads) {
      const double mc = cm[c];
      const int vc = cv[c];
      if (vc >= nb) continue;   // a wavefront with fewer than K tiles
      int r = 0;
      for (int e = 0; e < nc; ++e) {
        const int ve = cv[e];
        const double me = cm[e];
        r += ve < nb && (me > mc || (me == mc && ve < vc));
      }
      if (r < K) {
        rk[vc] = r;
        top[r] = vc;
      }
    }
    __syncthreads();
  } else {
    for (int v = t; v < nb; v += kThreads) {
      const double m = mass[v];
      int r = 0;
      for (int w = 0; w < nb; ++w) {
        const double x = mass[w];
        r += (x > m) || (x == m && w < v);
      }
      if (r < K) {
        rk[v] = r;
        top[r] = v;
      }
    }
    __syncthreads();
  }

  // step 10: inclusion probabilities of the residual.  With r_i the i-th
  // largest residual mass (rank ne + i) and S_i the sum of r_i and every
  // smaller one, k is the first i < m_sample with (m_sample - i) r_i <= S_i
  // (m_sample if none), lambda = (m_sample - k) / S_k; the residual's k
  // largest get pi = 1 and the rest lambda * mass.  S_i is the sum of the
  // tiles past rank K plus r_{m_sample-1} ... r_i.
  int k = 0;
  double lam = 0.0;
  if (capped) {
    double tail = 0.0;
    for (int v = t; v < nb; v += kThreads)
      if (rk[v] >= K) tail += mass[v];
    tail = block_sum(tail, red);
    if (t == 0) {
      double S = tail;
      cum[m_sample] = S;
      for (int i = m_sample - 1; i >= 0; --i) {
        S += mass[top[ne + i]];
        cum[i] = S;
      }
      int kk = m_sample;
      for (int i = 0; i < m_sample; ++i)
        if ((double)(m_sample - i) * mass[top[ne + i]] <= cum[i]) {
          kk = i;
          break;
        }
      k_s = kk;
      lam_s = (double)(m_sample - kk) / cum[kk];
    }
    __syncthreads();
    k = k_s;
    lam = lam_s;
  }
  auto pi_of = [&](int v) -> double { return (!capped || rk[v] < ne + k) ? 1.0 : lam * mass[v]; };

  // step 11: systematic PPS over the residual in ascending tile order
  for (int v = t; v < nb; v += kThreads) cum[v] = rk[v] < ne ? 0.0 : pi_of(v);
  __syncthreads();
  block_scan(cum, nb, red);
  const double uo = uoff[bh * G + g];
  for (int v = t; v < nb; v += kThreads) {
    const bool ex = rk[v] < ne;
    const double pv = pi_of(v);
    bool kept = ex;
    if (!ex) {
      // [lo, hi): the running sum before and after this tile (exact tiles add 0)
      const double hi = cum[v], lo = v > 0 ? cum[v - 1] : 0.0;
      const double klo = fmin(ceil(lo - uo), (double)m_sample), khi = fmin(ceil(hi - uo), (double)m_sample);
      kept = khi > klo;
    }
    keep[v] = kept ? 1 : 0;
    // step 13: Horvitz-Thompson weight as a log-weight
    lwv[v] = (kept && !ex && pv < 1.0) ? (float)(-log(pv)) : 0.f;
    if (pi_out) pi_out[(bh * G + g) * nb + v] = pv;
  }
  __syncthreads();
  for (int u = u0; u < u1; ++u) {
    const int64_t r = bh * nb + u;
    for (int v = t; v < nb; v += kThreads) {
      mask[r * nb + v] = keep[v];
      lw_map[r * nb + v] = v == u ? 0.f : lwv[v];
    }
  }
}

}  // namespace

extern "C" int bsa_segment_offsets(const int32_t *labels, int64_t BH, int64_t N, int32_t G, int32_t *seg_ptr,
                                   bsa_stream_t stream) {
  if (!labels || !seg_ptr || BH < 0 || N < 0 || G <= 0) return BSA_ERR_ARG;
  if (G > kMaxGroups || N >= (int64_t(1) << 31) || BH > 0x7fffffff) return BSA_ERR_UNSUPPORTED;
  if (BH == 0) return BSA_OK;
  hipLaunchKernelGGL(segment_offsets_kernel, dim3((unsigned)BH), dim3(kOffThreads), 0, bsa_hip_stream(stream),
                     labels, N, G, seg_ptr);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_segment_means(const void *x, const int64_t x_str[3], int32_t B, int32_t H, int64_t N, int32_t d,
                                 const int32_t *seg_ptr, int32_t G, int32_t seg_len, float *means,
                                 bsa_stream_t stream) {
  if (!x || !x_str || !means || B < 0 || H < 0 || N <= 0 || d <= 0) return BSA_ERR_ARG;
  if (seg_ptr ? G <= 0 : seg_len <= 0) return BSA_ERR_ARG;
  if (d % 8 || d > kMaxD || !bsa_aligned16(x)) return BSA_ERR_UNSUPPORTED;
  for (int i = 0; i < 3; ++i)
    if (x_str[i] < 0 || (x_str[i] & 7)) return BSA_ERR_ARG;
  if (x_str[2] < d) return BSA_ERR_ARG;
  const int64_t groups = seg_ptr ? G : (N + seg_len - 1) / seg_len;
  if (groups > 0x7fffffff) return BSA_ERR_UNSUPPORTED;
  if ((int64_t)B * H == 0) return BSA_OK;
  if ((int64_t)B * H > 65535) return BSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(segment_means_kernel, dim3((unsigned)groups, (unsigned)(B * H)), dim3(kThreads), 0,
                     bsa_hip_stream(stream), static_cast<const uint16_t *>(x), x_str[0], x_str[1], x_str[2], H, N, d,
                     seg_ptr, (int)groups, seg_len, means);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_is_sample(const float *qbar, const float *kbar, const int32_t *q_seg_ptr, const double *uoff,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t G, int64_t N, int32_t block, int32_t d,
                             int32_t m_exact, int32_t m_sample, float scale, uint8_t *mask, float *lw_map,
                             double *pi_out, bsa_stream_t stream) {
  if (!qbar || !kbar || !q_seg_ptr || !uoff || !mask || !lw_map) return BSA_ERR_ARG;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || G <= 0 || N <= 0 || block <= 0 || d <= 0) return BSA_ERR_ARG;
  if (m_exact < 0 || m_sample < 0) return BSA_ERR_ARG;
  const int64_t nb = (N + block - 1) / block;
  if (nb > kMaxTiles || d > kMaxD || G > 65535) return BSA_ERR_UNSUPPORTED;
  if ((int64_t)B * Hq > 65535) return BSA_ERR_UNSUPPORTED;
  if (B == 0) return BSA_OK;
  const double sc = scale > 0.f ? (double)scale : 1.0 / sqrt((double)d);
  hipLaunchKernelGGL(is_sample_kernel, dim3((unsigned)G, (unsigned)(B * Hq)), dim3(kThreads), 0,
                     bsa_hip_stream(stream), qbar, kbar, q_seg_ptr, uoff, Hq, Hkv, G, N, block, d, m_exact, m_sample,
                     sc, mask, lw_map, pi_out);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}
