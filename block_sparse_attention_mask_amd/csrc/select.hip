// Exact token-level KV selection for query groups (MC-Sparse, "The MC-Sparse
// Architecture" and Algorithm 1: at an anchor step a dense FlashAttention
// pass yields each query's log-sum-exp l_t; exact selection then recovers
// every attention probability exp(q_t . k_s * scale - l_t), sums it over the
// queries of a group, and keeps the K keys of largest summed mass, which the
// token-level sparse attention kernel consumes as the group's key list).
//
// Two kernels:
//
// group_mass -- one workgroup per (group, key chunk), eight wavefronts, two
//   per SIMD.  Wavefront w owns half w % 2 of the group's queries and the key
//   quarter w / 2 (32 keys) of every 128-key tile.  Key tiles stream through
//   four LDS stages by LDS DMA (buffer_load ... lds, 16-byte chunks of each
//   key row at XOR-swizzled positions), three tiles ahead, one barrier per
//   tile; both query halves read the same staged tile.  The scores of the
//   next tile are computed while the current tile's exponentials run.  S = Q K^T runs on 32x32x16 bf16 MFMA with the query fragments held
//   in registers for the whole chunk (A operand, one query row per lane) and
//   the key fragments read from LDS (B operand, one key column per lane), so
//   a lane ends with 16 query rows of one key column: p = exp2(s * c - l2_t) is
//   summed down the column in registers, the two lane halves are added with
//   one cross-lane exchange, and the two query halves meet in LDS, flushed
//   once per 1024 keys.  Summation order is fixed, so results are
//   deterministic.  Causal: keys past the group's last query are written as
//   zeros without being computed; tiles reaching past the group's first
//   query mask per element.
//
// topk_rows -- one workgroup per row, the row held in registers as
//   order-preserving 32-bit keys (E consecutive elements per thread).  The K-th largest key is found by a bitwise search from the top
//   bit (count of keys >= candidate, summed over the workgroup), then one
//   pair of workgroup scans over the counts of keys above it and equal to
//   it places every selected index: all keys above the threshold and the
//   lowest-indexed ties, written in ascending index order.
#include <type_traits>

#include "attn_common.h"

namespace bsa {
namespace sel {

struct MassParams {
  const uint16_t *q, *k;
  const float *lse;
  float *mass;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2;
  const int32_t *q_idx;
  int64_t rows;   // B * Hq * n_sets
  int64_t ldm;    // k1 - k0 (mass row length)
  int32_t sets, Hq, G, N;
  int32_t k0, k1, chunk;
  int32_t causal;
  float c;        // scale * log2(e)
};

constexpr int kSuper = 1024;      // keys per LDS flush (eight 128-key tiles)
constexpr int kStages = 4;        // K tiles staged in LDS
constexpr int kTileBytes = 128 * 128 * 2;

template <int BQ>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void group_mass(MassParams p) {
  constexpr int D = 128, KS = D / 16, QT = BQ / 64, HALF = BQ / 2;
  __shared__ __attribute__((aligned(1024))) uint8_t kt[kStages][kTileBytes];
  __shared__ float part[2][2][kSuper];   // [buffer][query half][key of the super tile]
  __shared__ int32_t qpos[BQ];
  __shared__ float ql2[BQ];
  __shared__ int tlo, thi;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qh = wave & 1, kq = wave >> 1;
  const int ln = lane & 31, hf = lane >> 5;
  const int64_t row = (int64_t)blockIdx.x % p.rows;
  const int split = (int)((int64_t)blockIdx.x / p.rows);
  const int64_t bh = row / p.sets;
  const int64_t b = bh / p.Hq, h = bh % p.Hq, g = h / p.G;
  const int N = p.N;

  if (tid == 0) { tlo = 0x7fffffff; thi = -1; }
  __syncthreads();
  if (tid < BQ) {
    const int t = p.q_idx[row * BQ + tid];
    const bool ok = t >= 0 && t < N;
    const float l = ok ? p.lse[bh * N + t] : 0.f;
    // an empty slot, or a query whose log-sum-exp is -inf or NaN, adds nothing
    const bool live = ok && l > -INFINITY;
    qpos[tid] = ok ? t : -1;
    ql2[tid] = live ? l * kLog2e : INFINITY;
    if (ok) { atomicMin(&tlo, t); atomicMax(&thi, t); }
  }
  __syncthreads();

  // this workgroup's keys [ka, kb); when causal, keys from kc on are zero
  const int ka = p.k0 + split * p.chunk;
  const int kb = min(p.k1, ka + p.chunk);
  const int kc = p.causal ? max(ka, min(kb, thi + 1)) : kb;
  const int tmin = tlo;
  float *mrow = p.mass + row * p.ldm - p.k0;

  const rsrc_t qrs = make_rsrc(p.q + b * p.qs0 + h * p.qs1, ((int64_t)(N - 1) * p.qs2 + D) * 2);
  const i32x4 krs = buffer_rsrc(p.k + b * p.ks0 + g * p.ks1, ((int64_t)(N - 1) * p.ks2 + D) * 2);

  // Q fragments (A operand): lane (ln, hf) of tile qt holds query slot
  // HALF qh + 32 qt + ln, dims 16 ks + 8 hf .. +7
  bf16x8 qa[QT][KS];
  float l2[QT][16];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int t = qpos[HALF * qh + 32 * qt + ln];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = t >= 0 ? (uint32_t)(((int64_t)t * p.qs2 + ks * 16 + hf * 8) * 2) : kOOR;
      qa[qt][ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
    }
    // accumulator element i of this lane is query row 8 (i / 4) + 4 hf + i % 4
#pragma unroll
    for (int i = 0; i < 16; ++i) l2[qt][i] = ql2[HALF * qh + 32 * qt + 8 * (i >> 2) + 4 * hf + (i & 3)];
  }

  // K tiles: copy I (0..31) of a tile fills LDS bytes [1024 I, 1024 I + 1024),
  // rows 4 I .. 4 I + 3; lane l writes row 4 I + l / 16 at chunk position
  // l % 16, which holds source chunk (l % 16) ^ (row mod 16).  Wavefront w
  // issues copies w, w + 8, w + 16, w + 24.  Keys at or past kc read zeros,
  // and so do the copies issued for tiles past the end, which keeps every
  // wavefront's count of copies in flight the same in every iteration.
  const uint32_t ks2b = (uint32_t)p.ks2 * 2;
  int crow[4];
  uint32_t coff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    crow[t] = 4 * (wave + 8 * t) + (lane >> 4);
    coff[t] = (uint32_t)crow[t] * ks2b + ((((uint32_t)lane & 15u) ^ ((uint32_t)crow[t] & 15u)) << 4);
  }
  auto lds_addr = [](const uint8_t *ptr) -> uint32_t {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)ptr;
  };
  auto issue = [&](int jt) {
    const int tile0 = ka + 128 * jt;
    const uint32_t dst = lds_addr(kt[jt & (kStages - 1)]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t off = tile0 + crow[t] < kc ? (uint32_t)tile0 * ks2b + coff[t] : kOOR;
      lds_copy16(krs, dst + 1024u * (wave + 8 * t), off, 0u);
    }
  };
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto flush = [&](int sup) {
    const int s0 = ka + kSuper * sup;
    const int send = min(kc, s0 + kSuper);
    for (int x = tid; x < send - s0; x += 512) mrow[s0 + x] = part[sup & 1][0][x] + part[sup & 1][1][x];
  };

  const int ntile = (kc - ka + 127) >> 7;
  const int r = 32 * kq + ln;   // this lane's key within a tile
  auto scores = [&](f32x16 (&acc)[QT], int jt) {   // S of tile jt from its LDS stage
    const uint8_t *kst = kt[jt & (kStages - 1)];
    bf16x8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = *reinterpret_cast<const bf16x8 *>(kst + r * 256 + (((2 * ks + hf) ^ (r & 15)) << 4));
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[qt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
        acc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[qt][ks], kf[ks], acc[qt], 0, 0, 0);
  };
  // Software pipeline: the scores of tile j+1 are computed (MFMA) in the same
  // basic block as the exponentials of tile j (VALU), so the two overlap
  // within each wavefront.  Tile j+4 is copied into the stage of tile j once
  // the barrier shows every wavefront has read it.
  f32x16 acc[QT], accn[QT];
#pragma unroll
  for (int jt = 0; jt < kStages; ++jt) issue(jt);
  if (ntile > 0) {
    __builtin_amdgcn_s_waitcnt(vm_lgkm0_wait_imm(4 * (kStages - 1)));
    barrier();
    scores(acc, 0);
  }
  for (int j = 0; j < ntile; ++j) {
    // tile j+1 has landed once at most the copies of tiles j+2, j+3 are in
    // flight; the barrier also marks the stage of tile j as read by all
    __builtin_amdgcn_s_waitcnt(vm_lgkm0_wait_imm(4 * (kStages - 2)));
    barrier();
    if (j > 0 && (j & 7) == 0) flush((j >> 3) - 1);
    issue(j + kStages);
    const int tile0 = ka + 128 * j;
    const int key = tile0 + r;
    auto step = [&](auto masked) {
      scores(accn, j + 1);   // past the end: a stage of zeros, result unused
      float col = 0.f;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = fmaf(acc[qt][i], p.c, -l2[qt][i]);
          if (decltype(masked)::value) {
            const int t = qpos[HALF * qh + 32 * qt + 8 * (i >> 2) + 4 * hf + (i & 3)];
            x = key > t ? -INFINITY : x;
          }
          col += __builtin_amdgcn_exp2f(x);
        }
      col += __shfl_xor(col, 32, 64);
      if (hf == 0) part[(j >> 3) & 1][qh][128 * (j & 7) + r] = col;
      if (!decltype(masked)::value) {
        __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);   // SGB: the K fragment reads
#pragma unroll
        for (int m = 0; m < QT * KS; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // SGB: one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // SGB: six VALU
        }
      }
    };
    if (p.causal && tile0 + 127 > tmin) step(std::integral_constant<bool, true>());
    else step(std::integral_constant<bool, false>());
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) acc[qt] = accn[qt];
  }
  // every copy (the ones past the end too) lands before the workgroup ends
  __builtin_amdgcn_s_waitcnt(0);
  barrier();
  if (ntile > 0) flush((ntile - 1) >> 3);
  // keys past the group's last query (causal) carry no mass
  for (int x = kc + tid; x < kb; x += 512) mrow[x] = 0.f;
}

// Order-preserving key of a float (larger float -> larger unsigned key);
// -0 and +0 share one key, denormals keep their order.  NaN inputs are not
// ranked meaningfully.
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Rows of up to 32768 keys: 1024 threads, E <= 32 keys each; longer rows (up
// to 77824): 512 threads with 152 keys each, in the larger register budget
// of two wavefronts per SIMD.
constexpr int kTopkLong = 152;

template <int E, int NT>
__global__ __attribute__((amdgpu_flat_work_group_size(NT, NT)))
void topk_rows(const float *x, int64_t ld, int n, int k, int32_t *idx, int vec) {
  constexpr int NWV = NT / 64;
  __shared__ int red[2][NWV];
  __shared__ int scan_gt[NWV], scan_eq[NWV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float *xr = x + row * ld;
  int32_t *out = idx + row * (int64_t)k;
  const int base = tid * E;

  // padding keys are 0, below every candidate, so they are never counted.
  // With 16-byte aligned rows each lane loads four keys at a time.
  uint32_t key[E];
  if (vec) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const int i = base + e;
      if (i + 3 < n) {
        const float4 v = *reinterpret_cast<const float4 *>(xr + i);
        key[e] = order_key(v.x); key[e + 1] = order_key(v.y);
        key[e + 2] = order_key(v.z); key[e + 3] = order_key(v.w);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) key[e + u] = i + u < n ? order_key(xr[i + u]) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) key[e] = base + e < n ? order_key(xr[base + e]) : 0u;
  }

  // threshold T: the largest key with at least k keys >= T
  uint32_t T = 0;
  if (k < n) {
    // Bits above the highest one in which the row's keys differ are the same
    // in every key (padding keys, 0, left out): a candidate with such a bit
    // counts all n keys or none, so T takes them as they are and the search
    // starts below them.
    uint32_t lo = ~0u, hi = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e]) { lo = min(lo, key[e]); hi = max(hi, key[e]); }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
      hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
    }
    if (lane == 0) { red[0][wave] = (int)lo; red[1][wave] = (int)hi; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      lo = min(lo, (uint32_t)red[0][w]);
      hi = max(hi, (uint32_t)red[1][w]);
    }
    __syncthreads();   // red is reused by the counting passes
    const uint32_t diff = lo ^ hi;
    const int top = diff ? 31 - __builtin_clz(diff) : -1;   // highest differing bit
    T = top < 0 ? hi : (top >= 31 ? 0u : hi & ~((2u << top) - 1u));
    int it = 0;
    for (int bit = top; bit >= 0; --bit, ++it) {
      const uint32_t cand = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) c += key[e] >= cand ? 1 : 0;
      c = bsa_wave_sum(c);
      if (lane == 0) red[it & 1][wave] = c;
      __syncthreads();
      int tot = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) tot += red[it & 1][w];
      if (tot >= k) T = cand;
      if (tot == k) break;   // exactly k keys >= T: no tie to break
    }
  }

  // all keys > T, then the lowest-indexed keys == T until k are taken
  int gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    gt += key[e] > T ? 1 : 0;
    eq += key[e] == T ? 1 : 0;
  }
  const int gt_inc = bsa_wave_incl_scan(gt, lane), eq_inc = bsa_wave_incl_scan(eq, lane);
  if (lane == 63) { scan_gt[wave] = gt_inc; scan_eq[wave] = eq_inc; }
  __syncthreads();
  int gt_before = gt_inc - gt, eq_before = eq_inc - eq, gt_total = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const int a = scan_gt[w], c = scan_eq[w];
    gt_total += a;
    if (w < wave) { gt_before += a; eq_before += c; }
  }
  const int need = k - gt_total;   // ties at T to take
  int pos = gt_before + min(eq_before, need);
  int tie = eq_before;
  // take-flags as bit masks, then a rolled walk over the set bits (ascending)
  constexpr int NB = (E + 31) / 32;
  uint32_t take[NB];
#pragma unroll
  for (int w = 0; w < NB; ++w) take[w] = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bool t = key[e] > T;
    if (key[e] == T) { t = tie < need; ++tie; }
    take[e >> 5] |= (t ? 1u : 0u) << (e & 31);
  }
#pragma unroll
  for (int w = 0; w < NB; ++w) {
    uint32_t m = take[w];
    while (m) {
      out[pos++] = base + 32 * w + __builtin_ctz(m);
      m &= m - 1u;
    }
  }
}

}  // namespace sel
}  // namespace bsa

extern "C" int bsa_group_mass(const bsa_mass_args *a, bsa_stream_t stream) {
  using namespace bsa;
  using namespace bsa::sel;
  if (!a) return BSA_ERR_ARG;
  if (!a->q || !a->k || !a->lse || !a->mass || !a->q_idx) return BSA_ERR_ARG;
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->N <= 0 || a->n_sets < 0) return BSA_ERR_ARG;
  if (a->Hq % a->Hkv) return BSA_ERR_ARG;
  if (a->d != 128 || (a->set_size != 64 && a->set_size != 128)) return BSA_ERR_UNSUPPORTED;
  if (a->k0 < 0 || a->k1 > a->N || a->k0 > a->k1) return BSA_ERR_ARG;
  if (!bsa_aligned16(a->q) || !bsa_aligned16(a->k)) return BSA_ERR_ARG;
  for (int i = 0; i < 3; ++i)
    if (a->q_str[i] < 0 || (a->q_str[i] & 7) || a->k_str[i] < 0 || (a->k_str[i] & 7)) return BSA_ERR_ARG;
  if (a->q_str[2] < a->d || a->k_str[2] < a->d) return BSA_ERR_ARG;
  const int64_t lim = int64_t(1) << 30;
  if (((a->N - 1) * a->q_str[2] + a->d) * 2 >= lim || ((a->N - 1) * a->k_str[2] + a->d) * 2 >= lim)
    return BSA_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)a->B * a->Hq * a->n_sets;
  const int64_t W = a->k1 - a->k0;
  if (rows == 0 || W == 0) return BSA_OK;
  // Split a row's key range only when a launch would otherwise hold too few
  // workgroups (K is re-read per group either way; splitting further only
  // adds per-workgroup set-up).
  const int64_t want = 4096;
  int64_t nsplit = (want + rows - 1) / rows;
  const int64_t max_split = (W + kSuper - 1) / kSuper;
  if (nsplit > max_split) nsplit = max_split;
  const int64_t chunk = ((W + nsplit - 1) / nsplit + kSuper - 1) / kSuper * kSuper;
  nsplit = (W + chunk - 1) / chunk;
  if (rows * nsplit >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  MassParams p;
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = static_cast<const uint16_t *>(a->k);
  p.lse = a->lse;
  p.mass = a->mass;
  p.qs0 = a->q_str[0]; p.qs1 = a->q_str[1]; p.qs2 = a->q_str[2];
  p.ks0 = a->k_str[0]; p.ks1 = a->k_str[1]; p.ks2 = a->k_str[2];
  p.q_idx = a->q_idx;
  p.rows = rows;
  p.ldm = W;
  p.sets = a->n_sets;
  p.Hq = a->Hq;
  p.G = a->Hq / a->Hkv;
  p.N = (int)a->N;
  p.k0 = (int)a->k0;
  p.k1 = (int)a->k1;
  p.chunk = (int)chunk;
  p.causal = a->causal ? 1 : 0;
  const float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->d);
  p.c = scale * kLog2e;
  hipStream_t s = bsa_hip_stream(stream);
  const dim3 grid((unsigned)(rows * nsplit));
  if (a->set_size == 64) hipLaunchKernelGGL(group_mass<64>, grid, dim3(512), 0, s, p);
  else hipLaunchKernelGGL(group_mass<128>, grid, dim3(512), 0, s, p);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}

extern "C" int bsa_topk_rows(const float *x, int64_t rows, int64_t n, int64_t ld, int32_t k, int32_t *idx,
                             bsa_stream_t stream) {
  using namespace bsa::sel;
  if (rows < 0 || n <= 0 || ld < n || k < 0) return BSA_ERR_ARG;
  if (rows == 0 || k == 0) return BSA_OK;
  if (!x || !idx) return BSA_ERR_ARG;
  if (n > 512 * kTopkLong) return BSA_ERR_UNSUPPORTED;
  if (rows >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  const int kk = k < n ? k : (int)n;
  const int nn = (int)n;
  // every row start 16-byte aligned: four-key loads (E is a multiple of 4)
  const int vec = (ld % 4 == 0 && bsa_aligned16(x)) ? 1 : 0;
  hipStream_t s = bsa_hip_stream(stream);
  const dim3 grid((unsigned)rows);
  if (n <= 4 * 1024) hipLaunchKernelGGL((topk_rows<4, 1024>), grid, dim3(1024), 0, s, x, ld, nn, kk, idx, vec);
  else if (n <= 8 * 1024) hipLaunchKernelGGL((topk_rows<8, 1024>), grid, dim3(1024), 0, s, x, ld, nn, kk, idx, vec);
  else if (n <= 16 * 1024) hipLaunchKernelGGL((topk_rows<16, 1024>), grid, dim3(1024), 0, s, x, ld, nn, kk, idx, vec);
  else if (n <= 32 * 1024) hipLaunchKernelGGL((topk_rows<32, 1024>), grid, dim3(1024), 0, s, x, ld, nn, kk, idx, vec);
  else hipLaunchKernelGGL((topk_rows<kTopkLong, 512>), grid, dim3(512), 0, s, x, ld, nn, kk, idx, vec);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}
