// Block-sparse softmax attention forward for CDNA4 (gfx950), V dim-major.
//
// Semantics as in InstaGen, section 3.1 Eq. (1)-(3) with the listed block's
// additive log-weight (Algorithm 1): for every query t of query block u,
// o_t = sum_s softmax_s(q_t.k_s / sqrt(d) + log w_v(s)) v_s over the keys of
// the KV blocks listed in row (b, h, u).  Keys past N and, when causal,
// keys s > t do not take part.
//
// Mapping to the hardware (one workgroup per CSR row, BLK queries):
//   * 2*BLK/32 wavefronts, two per SIMD.  Wavefront w owns the 32 queries of
//     group w % (BLK/32) and the key half w / (BLK/32) of every KV tile; the
//     two halves keep separate online-softmax states that are merged once
//     through LDS after the last tile.
//   * K tiles ([key][dim]) and V^T tiles ([dim][key], V stored dim-major in
//     HBM) are copied straight into LDS with buffer_load_dwordx4 ... lds.
//     Every LDS row is padded by one 16-byte slot, so 16 consecutive rows
//     start in 16 different bank groups (conflict-free 16-byte reads with
//     plain immediate offsets); the copy writes junk into the pad slots.
//     Source offsets are per-lane constants plus a per-tile scalar offset;
//     rows past the end of a buffer come back as zeros (range checking).
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16.  MFMA row m
//     of an S^T tile is mapped to key 16(m>>4) + 8((m>>2)&1) + 4((m>>3)&1) +
//     (m&3), so that the eight probabilities a lane holds per PV k-step are
//     eight consecutive keys and the matching V^T operand is one 16-byte read.
//   * Software pipeline, one barrier per tile: interval i computes
//     S(i+1) = K(i+1) Q^T in the same basic block as the exponentials of S(i)
//     (independent, so MFMA and VALU work interleave), then O += V(i) P(i).
//     K tiles and V tiles each rotate through two LDS stages, one tile apart:
//     during interval i the copies of K(i+2) and V(i+1) are in flight.
//   * Softmax in base 2, fp32; the running max is only raised (and O
//     rescaled) when a tile's max exceeds it by more than 8, which is exact
//     and leaves probabilities <= 2^8.
#include "attn_common.h"

namespace bsa {
namespace dimv {

template <int BLK, int D>
struct DCfg {
  static constexpr int NQG = BLK / 32;            // query groups of 32
  static constexpr int NW = 2 * NQG;              // wavefronts: query group x key half
  static constexpr int NT = 64 * NW;              // threads (= 4 BLK, the launch bound)
  static_assert(NT == 4 * BLK, "launch bound");
  static constexpr int MTW = BLK / 64;            // 32-key M tiles per wavefront per KV tile
  static constexpr int KS = D / 16;               // k-steps of K Q^T
  static constexpr int DT = D / 32;               // 32-dim M tiles of O^T
  static constexpr int KC = D / 8, KP = KC + 1;   // K rows: 16-byte chunks, padded pitch
  static constexpr int VC = BLK / 8, VP = VC + 1; // V^T rows: chunks, padded pitch
  static constexpr int NIK = BLK * KP / 64;       // 1 KB copies per K tile
  static constexpr int NIV = D * VP / 64;         // 1 KB copies per V^T tile
  static constexpr int NIKW = (NIK + NW - 1) / NW;
  static constexpr int NIVW = (NIV + NW - 1) / NW;
  static constexpr int MERGE_FLOATS = 64 * (DT * 16 + 2);  // per query group
  static constexpr int KBUF = NIK * 1024 > MERGE_FLOATS * 4 ? NIK * 1024 : MERGE_FLOATS * 4;
  static constexpr int VBUF = NIV * 1024 > MERGE_FLOATS * 4 ? NIV * 1024 : MERGE_FLOATS * 4;
  static constexpr int LIST = 1024;               // CSR entries staged in LDS at a time
  static_assert(BLK * KP % 64 == 0 && D * VP % 64 == 0, "whole copies per tile");
  static_assert(NQG <= 4, "one merge buffer per query group");
};

template <int BLK, int D, bool kCrm>
__device__ __forceinline__ void attn_dimv_body(const AttnParams &p, const int32_t *__restrict__ row_ptr,
                                               const int32_t *__restrict__ col, const float *__restrict__ lw,
                                               const int32_t *__restrict__ order,
                                               const int32_t *__restrict__ sperm, uint16_t *__restrict__ out,
                                               float *__restrict__ lse) {
  // The index arrays are read-only and never alias the outputs (restrict), so
  // their wave-uniform reads become scalar loads.
  using C = DCfg<BLK, D>;
  // K and V^T stages are separate objects, so the compiler can tell the
  // stage being filled by DMA from the stages being read.
  __shared__ __attribute__((aligned(1024))) uint8_t k0[C::KBUF], k1[C::KBUF], v0[C::VBUF], v1[C::VBUF];
  __shared__ int32_t lcol[C::LIST];
  __shared__ float lbias[C::LIST];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < C::NW);
  const int ln = lane & 31, hf = lane >> 5;
  const int qg = wave % C::NQG, kh = wave / C::NQG;
  const int32_t r = order ? order[blockIdx.x] : (int32_t)blockIdx.x;
  if (r < 0 || r >= p.R) return;   // a launch-table entry outside the rows computes nothing
  const int64_t bh = r / p.nQB;
  const int u = (int)(r - bh * p.nQB);
  const int64_t b = bh / p.Hq;
  const int h = (int)(bh - b * p.Hq);
  const int g = h / p.G;
  // every per-head extent is below 2^30 bytes, so token positions fit in 32 bits
  const int N = (int)p.N;
  // the row's list: entries [e0, e1) of col, or positions [0, e1) of the
  // walk over the row's CRM words
  int e0, e1;
  const uint32_t *crow = nullptr;
  if constexpr (kCrm) {
    crow = p.crm + (int64_t)r * p.crm_words;
    e0 = 0;
    // the first chunk is walked here; a row shorter than a chunk needs no
    // separate count
    const int seen = bsa_crm_walk(crow, p.crm_words, p.crm_tail, 0, C::LIST, lcol, wave, C::NW, lane);
    e1 = __builtin_amdgcn_readfirstlane(seen < C::LIST ? seen : bsa_crm_count(crow, p.crm_words, p.crm_tail, lane));
  } else {
    e0 = row_ptr[r];
    e1 = row_ptr[r + 1];
  }
  // KV blocks at or after mlim need the element mask: the partial last block
  // and, when causal, blocks from the diagonal on
  const int nfull = N / BLK;
  const int mlim = p.causal ? (u < nfull ? u : nfull) : nfull;
  const int qi = u * BLK + qg * 32 + ln;   // this lane's query position

  const rsrc_t qrs = make_rsrc(p.q + b * p.qs0 + h * p.qs1, ((int64_t)(N - 1) * p.qs2 + D) * 2);
  const rsrc_t krs = make_rsrc(p.k + b * p.ks0 + g * p.ks1, ((int64_t)(N - 1) * p.ks2 + D) * 2);
  const rsrc_t vrs = make_rsrc(p.v + b * p.vs0 + g * p.vs1, (int64_t)D * p.vs2 * 2);
  const uint32_t ks2b = (uint32_t)p.ks2 * 2, vs2b = (uint32_t)p.vs2 * 2;

  // Q^T fragment (B operand): lane (ln, hf) holds q[qrow][16 ks + 8 hf .. +7],
  // qrow the row of q holding query qi (through the gather permutation)
  const int qrow = (qi < N && p.gperm) ? p.gperm[bh * N + qi] : qi;
  const bool qok = qi < N && qrow >= 0 && qrow < N;
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = qok ? (uint32_t)(((int64_t)qrow * p.qs2 + ks * 16 + hf * 8) * 2) : kOOR;
    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  }

  // Per-lane source offsets of this wavefront's 1 KB copies (copy I = wave + NW t
  // writes LDS slots 64 I .. 64 I + 63, slot s = row * pitch + chunk).
  uint32_t kvo[C::NIKW], vvo[C::NIVW];
#pragma unroll
  for (int t = 0; t < C::NIKW; ++t) {
    const int s = (wave + C::NW * t) * 64 + lane;
    const int row = s / C::KP, c = s % C::KP;
    kvo[t] = (c < C::KC && row < BLK) ? (uint32_t)row * ks2b + c * 16 : kOOR;
  }
#pragma unroll
  for (int t = 0; t < C::NIVW; ++t) {
    const int s = (wave + C::NW * t) * 64 + lane;
    const int row = s / C::VP, c = s % C::VP;
    vvo[t] = (c < C::VC && row < D) ? (uint32_t)row * vs2b + c * 16 : kOOR;
  }
  // scalar offset of list entry i's tile, or one past every buffer for a
  // block index outside the rows (then the tile reads as zeros)
  auto k_soff = [&](int i) -> uint32_t {
    const uint32_t vb = (uint32_t)lcol[i];
    return vb < (uint32_t)p.nQB ? vb * BLK * ks2b : kOOR;   // rows >= N read as zeros
  };
  auto v_soff = [&](int i) -> uint32_t {
    const uint32_t vb = (uint32_t)lcol[i];
    return vb < (uint32_t)p.nQB ? vb * BLK * 2 : kOOR;
  };
  // The LDS destination of copy t is stage + 1024 (wave + NW t); all but the
  // last copy of every wavefront exist (NW (NIKW - 1) < NIK).  The wave offset
  // passes through an empty asm so that the per-copy addresses are formed at
  // each issue (one scalar add each) instead of occupying scalar registers for
  // the whole loop.
  auto issue_k = [&](int i, uint8_t *dst) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(k_soff(i));
    int wo = wave * 1024;
    asm volatile("" : "+s"(wo));
#pragma unroll
    for (int t = 0; t < C::NIKW; ++t)
      if (t < C::NIKW - 1 || wave + C::NW * t < C::NIK)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(dst + wo + C::NW * 1024 * t), 16, kvo[t], so, 0, 0);
  };
  auto issue_v = [&](int i, uint8_t *dst) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(v_soff(i));
    int wo = wave * 1024;
    asm volatile("" : "+s"(wo));
#pragma unroll
    for (int t = 0; t < C::NIVW; ++t)
      if (t < C::NIVW - 1 || wave + C::NW * t < C::NIV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(dst + wo + C::NW * 1024 * t), 16, vvo[t], so, 0, 0);
  };

  // LDS read bases (immediate offsets do the rest)
  int kb[C::MTW];
#pragma unroll
  for (int jj = 0; jj < C::MTW; ++jj) kb[jj] = (32 * (kh * C::MTW + jj) + key_of_row(ln)) * C::KP * 16 + hf * 16;
  const int vbase = ln * C::VP * 16 + hf * 16;
  const int ob = 32 * kh * C::MTW + 8 * hf;   // key offset of this lane's first score row

  auto qk = [&](f32x16 (&s)[C::MTW], const uint8_t *kt) {
#pragma unroll
    for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[jj][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj) {
        const uint4 a = *reinterpret_cast<const uint4 *>(kt + kb[jj] + ks * 32);
        s[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[jj], 0, 0, 0);
      }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  f32x16 sa[C::MTW], sb[C::MTW];

  // One pipeline interval: softmax of S(i) (in sc) overlapped with
  // S(i+1) = K(i+1) Q^T (into sn), then O += V(i) P(i).
  auto interval = [&](int i, f32x16 (&sc)[C::MTW], f32x16 (&sn)[C::MTW], const uint8_t *kt_next,
                      const uint8_t *vt) {
    const uint32_t vb = (uint32_t)lcol[i];
    const float bias = lbias[i];
    if (vb >= (uint32_t)mlim) {
      // keys past N (last block) and, when causal, keys after the query; a
      // block index outside the rows masks every key.  Element e of M tile
      // jj holds key offset ob + 32 jj + 16 (e >> 3) + (e & 7) in the block.
      const int vbc = vb < (uint32_t)p.nQB ? (int)vb : p.nQB;
      const int kbase = vbc * BLK;
      const int lim_n = N - kbase > BLK ? BLK : (N - kbase < 0 ? 0 : N - kbase);   // offsets >= lim_n: padding
      const int lc = p.causal ? qi - kbase + 1 : BLK;                               // offsets >= lc: after the query
      const int lim = (lc < lim_n ? lc : lim_n) - ob;
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * jj + 16 * (e >> 3) + (e & 7) >= lim) sc[jj][e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[jj][e]);
    mx = halves_max(mx);
    const float m_tile = (mx == -INFINITY) ? -INFINITY : fmaf(mx, p.c, bias);
    if (__any(m_tile > m_run + kTau)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
      m_run = m_new;
    }
    const float nb = bias - (m_run == -INFINITY ? 0.f : m_run);
    bf16x8 pb[C::MTW][2];
    auto exps = [&]() {
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float pv[8];
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) pv[e8] = __builtin_amdgcn_exp2f(fmaf(sc[jj][8 * s2 + e8], p.c, nb));
          l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
          pb[jj][s2] = __builtin_bit_cast(bf16x8, make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                                                             cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7])));
        }
    };
    // S(i+1) is computed unconditionally so that the MFMAs and the
    // exponentials share one basic block; after a row's last tile it reads a
    // stale stage and is never used
    qk(sn, kt_next);
    exps();
#pragma unroll
    for (int jj = 0; jj < C::MTW; ++jj) {
      const int j = kh * C::MTW + jj;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const uint4 a = *reinterpret_cast<const uint4 *>(vt + vbase + dt * 32 * C::VP * 16 + (4 * j + 2 * s2) * 16);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[jj][s2], o[dt], 0, 0, 0);
        }
    }
  };

  for (int c0 = e0; c0 < e1; c0 += C::LIST) {
    const int n = e1 - c0 < C::LIST ? e1 - c0 : C::LIST;
    if constexpr (kCrm) {
      if (c0 > 0) bsa_crm_walk(crow, p.crm_words, p.crm_tail, c0, n, lcol, wave, C::NW, lane);
      for (int i = tid; i < n; i += C::NT) lbias[i] = 0.f;
    } else {
      for (int i = tid; i < n; i += C::NT) {
        lcol[i] = col[c0 + i];
        lbias[i] = lw ? lw[c0 + i] * kLog2e : 0.f;
      }
    }
    __syncthreads();
    // prologue: K(0), V(0), K(1) resident, then S(0)
    issue_k(0, k0);
    issue_v(0, v0);
    if (n > 1) issue_k(1, k1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    qk(sa, k0);
    // the first interval refills k0 with K(2): every wavefront must be done
    // reading K(0) first
    if (n > 2) __syncthreads();
    for (int i = 0; i < n; i += 2) {
      // interval i (even): reads K(i+1) in k1, V(i) in v0; fills k0 <- K(i+2), v1 <- V(i+1)
      if (i + 2 < n) issue_k(i + 2, k0);
      if (i + 1 < n) issue_v(i + 1, v1);
      interval(i, sa, sb, k1, v0);
      __builtin_amdgcn_s_waitcnt(0);   // this wavefront's copies have landed
      __syncthreads();                 // ... and everyone's; the stages read above are free
      if (i + 1 >= n) break;
      // interval i+1 (odd): reads K(i+2) in k0, V(i+1) in v1; fills k1 <- K(i+3), v0 <- V(i+2)
      if (i + 3 < n) issue_k(i + 3, k1);
      if (i + 2 < n) issue_v(i + 2, v0);
      interval(i + 1, sb, sa, k0, v1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // merge the two key halves of every query group, normalise, store
  const float l_w = halves_sum(l_run);
  // after the last barrier no tile is read any more: one buffer per query group
  uint8_t *const mbuf = qg == 0 ? (uint8_t *)k0 : qg == 1 ? (uint8_t *)v0 : qg == 2 ? (uint8_t *)k1 : (uint8_t *)v1;
  float *scratch = reinterpret_cast<float *>(mbuf);
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<f32x4 *>(scratch + ((dt * 4 + i4) * 64 + lane) * 4) =
            f32x4{o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
    scratch[C::DT * 16 * 64 + lane] = m_run;
    scratch[C::DT * 16 * 64 + 64 + lane] = l_w;
  }
  __syncthreads();
  if (kh != 0) return;
  const float m2 = scratch[C::DT * 16 * 64 + lane];
  const float l2 = scratch[C::DT * 16 * 64 + 64 + lane];
  const float m = fmaxf(m_run, m2);
  const float a1 = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
  const float a2 = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - m);
  const float l_tot = l_w * a1 + l2 * a2;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int oi = (qi < N && sperm) ? sperm[bh * N + qi] : qi;
  if (qi < N && oi >= 0 && oi < N) {
    uint16_t *ob16 = out + b * p.os0 + h * p.os1 + (int64_t)oi * p.os2;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 o2 = *reinterpret_cast<const f32x4 *>(scratch + ((dt * 4 + i4) * 64 + lane) * 4);
        const float x0 = (o[dt][4 * i4] * a1 + o2[0] * a2) * inv;
        const float x1 = (o[dt][4 * i4 + 1] * a1 + o2[1] * a2) * inv;
        const float x2 = (o[dt][4 * i4 + 2] * a1 + o2[2] * a2) * inv;
        const float x3 = (o[dt][4 * i4 + 3] * a1 + o2[3] * a2) * inv;
        *reinterpret_cast<uint2 *>(ob16 + 32 * dt + 8 * i4 + 4 * hf) =
            make_uint2(cvt_pk_bf16(x0, x1), cvt_pk_bf16(x2, x3));
      }
    if (lse && hf == 0) lse[bh * N + oi] = l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// One plain kernel per tile shape and list format (the body is a
// force-inlined template).
#define BSA_DIMV_KERNEL(NAME, BLK, D, CRM)                                                          \
  __global__ __attribute__((amdgpu_flat_work_group_size(4 * BLK, 4 * BLK), amdgpu_waves_per_eu(2, 2))) \
  void NAME(const AttnParams p, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col, \
            const float *__restrict__ lw, const int32_t *__restrict__ order,                         \
            const int32_t *__restrict__ sperm, uint16_t *__restrict__ out, float *__restrict__ lse) { \
    attn_dimv_body<BLK, D, CRM>(p, row_ptr, col, lw, order, sperm, out, lse);                      \
  }
BSA_DIMV_KERNEL(attn_dimv_128_128, 128, 128, false)
BSA_DIMV_KERNEL(attn_dimv_128_64, 128, 64, false)
BSA_DIMV_KERNEL(attn_dimv_64_128, 64, 128, false)
BSA_DIMV_KERNEL(attn_dimv_64_64, 64, 64, false)
BSA_DIMV_KERNEL(attn_dimv_crm_64_128, 64, 128, true)
BSA_DIMV_KERNEL(attn_dimv_crm_64_64, 64, 64, true)
#undef BSA_DIMV_KERNEL

}  // namespace dimv

hipError_t launch_attn_dimv(const AttnParams &p, int block, int d, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), t(4 * block);
#define BSA_ARGS p, p.row_ptr, p.col, p.lw, p.order, p.sperm, p.o, p.lse
  if (p.crm) {
    if (block != 64) return hipErrorInvalidValue;
    if (d == 128) hipLaunchKernelGGL(dimv::attn_dimv_crm_64_128, g, t, 0, s, BSA_ARGS);
    else hipLaunchKernelGGL(dimv::attn_dimv_crm_64_64, g, t, 0, s, BSA_ARGS);
  } else if (block == 128 && d == 128) hipLaunchKernelGGL(dimv::attn_dimv_128_128, g, t, 0, s, BSA_ARGS);
  else if (block == 128) hipLaunchKernelGGL(dimv::attn_dimv_128_64, g, t, 0, s, BSA_ARGS);
  else if (d == 128) hipLaunchKernelGGL(dimv::attn_dimv_64_128, g, t, 0, s, BSA_ARGS);
  else hipLaunchKernelGGL(dimv::attn_dimv_64_64, g, t, 0, s, BSA_ARGS);
#undef BSA_ARGS
  return hipGetLastError();
}

}  // namespace bsa
