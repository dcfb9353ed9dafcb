// Block-sparse softmax attention forward for CDNA4 (gfx950), V token-major.
//
// Semantics (InstaGen, section 3.1 Eq. (1)-(3) and Algorithm 1): for every
// query t of query block u, o_t = sum_s softmax_s(q_t.k_s / sqrt(d) + log w_v(s)) v_s
// over the keys s of the KV blocks v listed in row (b, h, u) of the CSR,
// with log w the listed block's additive log-weight.  Keys past N in the last
// block and, when causal, keys s > t do not take part.
//
// One workgroup computes one row: a BLK-query block against its listed BLK-key
// blocks, FlashAttention-style (online softmax, fp32 running max and sum).
//
//   * BLK/32 wavefronts; wavefront w owns queries w*32 .. w*32+31.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: the key tile is the A operand (from LDS), the
//     query fragment is the B operand (held in VGPRs for the whole row).  In
//     the 32x32 accumulator layout every lane then holds one query column, so
//     the row max and row sum are in-lane reductions plus one exchange with
//     the lane 32 away.
//   * O^T = V^T P^T: the probabilities stay in registers as the B operand
//     (converted to bf16 in place: the accumulator's key order is reused as
//     the MFMA's contraction order), V^T comes from LDS.  V is transposed on
//     its way into LDS, 4 keys x 8 dims per thread, written as 8-byte rows.
//   * K and V tiles are double-buffered in LDS; tile e+2's global loads are in
//     flight in registers while tile e is computed, so one barrier per tile.
//   * LDS rows are XOR-swizzled so that the 16-byte K reads and 8-byte V^T
//     reads of a wavefront fall into distinct banks.
//   * The softmax works in base 2: scores are scaled by scale*log2(e) with
//     one FMA that also subtracts the running max and adds the block's
//     log-weight (also times log2(e)); v_exp_f32 is a native 2^x.
#include "attn_common.h"

namespace bsa {
namespace {

template <int BLK, int D>
struct Cfg {
  static constexpr int NW = BLK / 32;              // wavefronts
  static constexpr int NT = NW * 64;               // threads
  static constexpr int MT = BLK / 32;              // 32-key M tiles of S^T
  static constexpr int KS = D / 16;                // k-steps of Q K^T
  static constexpr int DT = D / 32;                // 32-dim M tiles of O^T
  static constexpr int KCH = D / 8;                // 16-byte chunks per K row
  static constexpr int K_LOADS = BLK * KCH / NT;   // 16-byte K loads per thread per tile
  static constexpr int VSL = BLK / 4;              // 8-byte slots (4 keys) per V^T row
  static constexpr int V_UNITS = (BLK / 4) * (D / 8) / NT;  // 4-key x 8-dim units per thread
  static_assert(K_LOADS * NT == BLK * KCH, "K tile split");
  static_assert(V_UNITS * NT == (BLK / 4) * (D / 8), "V tile split");
};

// K tile: row = key, 16-byte chunk swizzle.
template <int KCH>
__device__ __forceinline__ int k_swz(int row) {
  return KCH == 16 ? (row & 15) : ((row >> 1) & 7);
}
// V^T tile: row = head dim, 8-byte slot swizzle.
template <int VSL>
__device__ __forceinline__ int v_swz(int row) {
  return (row ^ (row >> 3)) & (VSL - 1);
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }


template <int BLK, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(BLK * 2, BLK * 2), amdgpu_waves_per_eu(1, 1)))
void attn_tokv_kernel(const AttnParams p) {
  using C = Cfg<BLK, D>;
  __shared__ uint4 lds_k[2][BLK * C::KCH];
  __shared__ uint2 lds_v[2][D * C::VSL];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 31, hf = lane >> 5;
  const int32_t r = p.order ? p.order[blockIdx.x] : (int32_t)blockIdx.x;
  if (r < 0 || r >= p.R) return;  // a launch table entry outside the rows computes nothing
  const int64_t bh = r / p.nQB;
  const int u = (int)(r - bh * p.nQB);
  const int64_t b = bh / p.Hq;
  const int h = (int)(bh - b * p.Hq);
  const int g = h / p.G;
  const int64_t N = p.N;
  const uint16_t *qb = p.q + b * p.qs0 + h * p.qs1;
  const uint16_t *kb = p.k + b * p.ks0 + g * p.ks1;
  const uint16_t *vb = p.v + b * p.vs0 + g * p.vs1;
  const int e0 = p.row_ptr[r], e1 = p.row_ptr[r + 1];
  const int64_t qi = (int64_t)u * BLK + wave * 32 + ln;  // this lane's query position

  // Q^T fragment (B operand): lane (ln, hf) holds q[qrow][16 ks + 8 hf .. +7],
  // qrow the row of q holding query qi (through the gather permutation).
  const int64_t qrow = (qi < N && p.gperm) ? (int64_t)p.gperm[bh * N + qi] : qi;
  const bool qok = qi < N && qrow >= 0 && qrow < N;
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (qok) x = ld16(qb + qrow * p.qs2 + ks * 16 + hf * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  uint4 kst[C::K_LOADS];
  uint4 vst[C::V_UNITS][4];

  auto gload = [&](int e) {
    const int64_t key0 = (int64_t)(uint32_t)p.col[e] * BLK;  // out-of-range entries load nothing
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int c = i * C::NT + tid;
      const int row = c / C::KCH, cc = c % C::KCH;
      const int64_t key = key0 + row;
      kst[i] = make_uint4(0, 0, 0, 0);
      if (key < N) kst[i] = ld16(kb + key * p.ks2 + cc * 8);
    }
#pragma unroll
    for (int i = 0; i < C::V_UNITS; ++i) {
      const int c = i * C::NT + tid;
      const int dch = c % (D / 8), kg = c / (D / 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t key = key0 + kg * 4 + j;
        vst[i][j] = make_uint4(0, 0, 0, 0);
        if (key < N) vst[i][j] = ld16(vb + key * p.vs2 + dch * 8);
      }
    }
  };

  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int c = i * C::NT + tid;
      const int row = c / C::KCH, cc = c % C::KCH;
      lds_k[buf][row * C::KCH + (cc ^ k_swz<C::KCH>(row))] = kst[i];
    }
#pragma unroll
    for (int i = 0; i < C::V_UNITS; ++i) {
      const int c = i * C::NT + tid;
      const int dch = c % (D / 8), kg = c / (D / 8);
      const uint32_t w0[4] = {vst[i][0].x, vst[i][0].y, vst[i][0].z, vst[i][0].w};
      const uint32_t w1[4] = {vst[i][1].x, vst[i][1].y, vst[i][1].z, vst[i][1].w};
      const uint32_t w2[4] = {vst[i][2].x, vst[i][2].y, vst[i][2].z, vst[i][2].w};
      const uint32_t w3[4] = {vst[i][3].x, vst[i][3].y, vst[i][3].z, vst[i][3].w};
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int rlo = dch * 8 + 2 * qd, rhi = rlo + 1;  // head-dim rows
        lds_v[buf][rlo * C::VSL + (kg ^ v_swz<C::VSL>(rlo))] =
            make_uint2(pack_lo(w0[qd], w1[qd]), pack_lo(w2[qd], w3[qd]));
        lds_v[buf][rhi * C::VSL + (kg ^ v_swz<C::VSL>(rhi))] =
            make_uint2(pack_hi(w0[qd], w1[qd]), pack_hi(w2[qd], w3[qd]));
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;

  if (e0 < e1) {
    gload(e0);
    lstore(0);
  }
  if (e0 + 1 < e1) gload(e0 + 1);
  __syncthreads();

  for (int e = e0; e < e1; ++e) {
    const int buf = (e - e0) & 1;
    if (e + 1 < e1) lstore(buf ^ 1);
    if (e + 2 < e1) gload(e + 2);

    const int64_t vblk = (int64_t)(uint32_t)p.col[e];
    const float bias = p.lw ? p.lw[e] * kLog2e : 0.f;

    // S^T = K Q^T for the BLK keys of this tile
    f32x16 s[C::MT];
#pragma unroll
    for (int j = 0; j < C::MT; ++j) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[j][i] = 0.f;
      const int row = 32 * j + ln;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const uint4 a = lds_k[buf][row * C::KCH + ((2 * ks + hf) ^ k_swz<C::KCH>(row))];
        s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[j], 0, 0, 0);
      }
    }

    // tail keys and causal masking (uniform branch per workgroup)
    const int64_t kbase = vblk * BLK;
    if (kbase + BLK > N || (p.causal && vblk >= u)) {
#pragma unroll
      for (int j = 0; j < C::MT; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = kbase + 32 * j + (i >> 2) * 8 + hf * 4 + (i & 3);
          if (key >= N || (p.causal && key > qi)) s[j][i] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < C::MT; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[j][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_tile = (mx == -INFINITY) ? -INFINITY : fmaf(mx, p.c, bias);
    const float m_new = fmaxf(m_run, m_tile);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    const float nb = bias - m_use;

#pragma unroll
    for (int j = 0; j < C::MT; ++j) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float pv[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          pv[e8] = __builtin_amdgcn_exp2f(fmaf(s[j][8 * s2 + e8], p.c, nb));
          l_run += pv[e8];
        }
        const uint4 pk = make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                                    cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7]));
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
        const int sl1 = 8 * j + 4 * s2 + hf, sl2 = sl1 + 2;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const int row = 32 * dt + ln;
          const uint2 a1 = lds_v[buf][row * C::VSL + (sl1 ^ v_swz<C::VSL>(row))];
          const uint2 a2 = lds_v[buf][row * C::VSL + (sl2 ^ v_swz<C::VSL>(row))];
          const uint4 a = make_uint4(a1.x, a1.y, a2.x, a2.y);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb, oacc[dt], 0, 0, 0);
        }
      }
    }
    m_run = m_new;
    __syncthreads();
  }

  // epilogue: O = acc / l, bf16 round-to-nearest-even; LSE in natural log
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t oi = (qi < N && p.sperm) ? (int64_t)p.sperm[bh * N + qi] : qi;
  if (qi < N && oi >= 0 && oi < N) {
    uint16_t *ob = p.o + b * p.os0 + h * p.os1 + oi * p.os2;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const uint2 w = make_uint2(cvt_pk_bf16(oacc[dt][4 * i4] * inv, oacc[dt][4 * i4 + 1] * inv),
                                   cvt_pk_bf16(oacc[dt][4 * i4 + 2] * inv, oacc[dt][4 * i4 + 3] * inv));
        *reinterpret_cast<uint2 *>(ob + 32 * dt + 8 * i4 + 4 * hf) = w;
      }
    if (p.lse && hf == 0)
      p.lse[bh * N + oi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_attn_tokv(const AttnParams &p, int block, int d, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid);
  if (block == 128 && d == 128) hipLaunchKernelGGL((attn_tokv_kernel<128, 128>), g, dim3(256), 0, s, p);
  else if (block == 128) hipLaunchKernelGGL((attn_tokv_kernel<128, 64>), g, dim3(256), 0, s, p);
  else if (d == 128) hipLaunchKernelGGL((attn_tokv_kernel<64, 128>), g, dim3(128), 0, s, p);
  else hipLaunchKernelGGL((attn_tokv_kernel<64, 64>), g, dim3(128), 0, s, p);
  return hipGetLastError();
}

}  // namespace bsa
