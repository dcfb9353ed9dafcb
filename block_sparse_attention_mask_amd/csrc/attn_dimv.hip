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
//     through LDS after the last tile.  Two resident wavefronts per SIMD let
//     one issue MFMAs while the other runs its softmax.
//   * K tiles ([key][dim]) and V^T tiles ([dim][key], V stored dim-major in
//     HBM) are copied straight into LDS with buffer_load_dwordx4 ... lds:
//     no register staging, and rows past the end of a buffer come back as
//     zeros (buffer range checking), so there are no branches on loads.
//     Two LDS stages: tile e+1 streams in while tile e is computed.
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16.  MFMA row m
//     of an S^T tile is mapped to key 16(m>>4) + 8((m>>2)&1) + 4((m>>3)&1) +
//     (m&3), which makes the eight probabilities a lane holds per PV k-step
//     eight consecutive keys; the matching V^T operand is then one 16-byte LDS
//     read, as is every K operand.
//   * LDS rows are 16-byte-chunk XOR-swizzled; the DMA source addresses carry
//     the inverse swizzle, so reads of 16 consecutive rows hit distinct banks.
//   * Softmax in base 2, fp32; the running max is only raised (and O
//     rescaled) when a tile's max exceeds it by more than 8, which is exact
//     and leaves probabilities <= 2^8.
#include "attn_common.h"

namespace bsa {
namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;  // >= every num_records used here
constexpr float kTau = 8.0f;             // lazy-rescale threshold (log2 units)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16-byte-chunk swizzle of an LDS row with CPR chunks.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  return CPR == 16 ? (row & 15) : ((row >> 1) & 7);
}

// Key (within a 32-key M tile) held by MFMA row m of S^T.
__device__ __forceinline__ int key_of_row(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

template <int BLK, int D>
struct DCfg {
  static constexpr int NQG = BLK / 32;            // query groups of 32
  static constexpr int NW = 2 * NQG;              // wavefronts: query group x key half
  static constexpr int NT = 64 * NW;              // threads
  static constexpr int MTW = BLK / 64;            // 32-key M tiles per wavefront per KV tile
  static constexpr int KS = D / 16;               // k-steps of K Q^T
  static constexpr int DT = D / 32;               // 32-dim M tiles of O^T
  static constexpr int KCPR = D / 8;              // 16-byte chunks per K row
  static constexpr int VCPR = BLK / 8;            // 16-byte chunks per V^T row
  static constexpr int TILE = BLK * D * 2;        // bytes of one K tile (= one V^T tile)
  static constexpr int DMA_PER_WAVE = TILE / 1024 / NW;
  static constexpr int K_ROWS_PER_DMA = 1024 / (D * 2);
  static constexpr int V_ROWS_PER_DMA = 1024 / (BLK * 2);
  static constexpr int MERGE_FLOATS = 64 * (DT * 16 + 2);   // per query group
  static constexpr int BUF = TILE > MERGE_FLOATS * 4 ? TILE : MERGE_FLOATS * 4;   // bytes per LDS buffer
  static constexpr int LIST = 1024;               // CSR entries staged in LDS at a time
  static_assert(DMA_PER_WAVE * NW * 1024 == TILE, "tile split");
  static_assert(NQG <= 4, "one merge buffer per query group");
};

template <int BLK, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(DCfg<BLK, D>::NT, DCfg<BLK, D>::NT),
                          amdgpu_waves_per_eu(2, 2)))
void attn_dimv_kernel(const AttnParams p, const int32_t *__restrict__ row_ptr,
                      const int32_t *__restrict__ col, const float *__restrict__ lw,
                      const int32_t *__restrict__ order, const int32_t *__restrict__ sperm,
                      uint16_t *__restrict__ out, float *__restrict__ lse) {
  // The index arrays are read-only and never alias the outputs (restrict), so
  // their wave-uniform reads become scalar loads that do not share the vector
  // memory counter with the in-flight tile copies.
  using C = DCfg<BLK, D>;
  // two LDS stages; separate objects so that the compiler can tell the stage
  // being filled by DMA from the stage being read
  __shared__ __attribute__((aligned(1024))) uint8_t k0[C::BUF], v0[C::BUF], k1[C::BUF], v1[C::BUF];
  // the row's KV-block list and log-weights, staged so that the loop reads
  // them from LDS instead of waiting on memory
  __shared__ int32_t lcol[C::LIST];
  __shared__ float lbias[C::LIST];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 31, hf = lane >> 5;
  const int qg = wave % C::NQG, kh = wave / C::NQG;
  const int32_t r = order ? order[blockIdx.x] : (int32_t)blockIdx.x;
  if (r < 0 || r >= p.R) return;   // a launch-table entry outside the rows computes nothing
  const int64_t bh = r / p.nQB;
  const int u = (int)(r - bh * p.nQB);
  const int64_t b = bh / p.Hq;
  const int h = (int)(bh - b * p.Hq);
  const int g = h / p.G;
  const int64_t N = p.N;
  const int e0 = row_ptr[r], e1 = row_ptr[r + 1];
  const int64_t qi = (int64_t)u * BLK + qg * 32 + ln;   // this lane's query position

  const rsrc_t qrs = make_rsrc(p.q + b * p.qs0 + h * p.qs1, ((N - 1) * p.qs2 + D) * 2);
  const rsrc_t krs = make_rsrc(p.k + b * p.ks0 + g * p.ks1, ((N - 1) * p.ks2 + D) * 2);
  const rsrc_t vrs = make_rsrc(p.v + b * p.vs0 + g * p.vs1, (int64_t)D * p.vs2 * 2);

  // Q^T fragment (B operand): lane (ln, hf) holds q[qi][16 ks + 8 hf .. +7]
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = qi < N ? (uint32_t)((qi * p.qs2 + ks * 16 + hf * 8) * 2) : kOutOfRange;
    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  }

  // Stream tile e (its K rows and V^T rows) into LDS stage `st`.
  const uint32_t ks2b = (uint32_t)p.ks2 * 2, vs2b = (uint32_t)p.vs2 * 2;
  const int32_t n32 = (int32_t)(N < INT32_MAX ? N : INT32_MAX);
  auto issue_tile = [&](int i, uint8_t *kdst, uint8_t *vdst) {
    // an out-of-range block index reads nothing (all rows out of range)
    const uint32_t vb = (uint32_t)lcol[i];
    const int32_t key0 = (int32_t)((vb < (uint32_t)p.nQB ? vb : (uint32_t)p.nQB) * BLK);
    const bool inside = vb < (uint32_t)p.nQB;
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
      const int I = wave * C::DMA_PER_WAVE + i;
      {
        const int row = I * C::K_ROWS_PER_DMA + lane / C::KCPR;
        const int cc = (lane % C::KCPR) ^ swz<C::KCPR>(row);
        const int32_t key = key0 + row;
        const uint32_t off0 = (uint32_t)(key < n32 ? key : 0) * ks2b + cc * 16;
        const uint32_t off = key < n32 ? off0 : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(kdst + I * 1024), 16, off, 0, 0, 0);
      }
      {
        const int row = I * C::V_ROWS_PER_DMA + lane / C::VCPR;   // head-dim row
        const int cc = (lane % C::VCPR) ^ swz<C::VCPR>(row);
        const uint32_t off = inside ? (uint32_t)row * vs2b + (uint32_t)key0 * 2 + cc * 16 : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(vdst + I * 1024), 16, off, 0, 0, 0);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  auto compute_tile = [&](int i, const uint8_t *kt, const uint8_t *vt) {
      const int64_t vblk = (int64_t)(uint32_t)lcol[i];
      const float bias = lbias[i];

      // S^T = K Q^T for this wavefront's BLK/2 keys
      f32x16 s[C::MTW];
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[jj][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj) {
          const int row = 32 * (kh * C::MTW + jj) + key_of_row(ln);
          const int ch = (2 * ks + hf) ^ swz<C::KCPR>(row);
          const uint4 a = *reinterpret_cast<const uint4 *>(kt + row * (D * 2) + ch * 16);
          s[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[jj], 0, 0, 0);
        }
      }

      // keys past N (last block) and, when causal, keys after the query
      const int64_t kbase = vblk * BLK;
      if (kbase + BLK > N || (p.causal && vblk >= u)) {
        const int64_t ln_ = N - kbase;
        const int lim_n = ln_ < 0 ? 0 : (ln_ > BLK ? BLK : (int)ln_);   // offsets >= lim_n are padding
        const int64_t lc_ = p.causal ? qi - kbase : (int64_t)BLK;
        const int lim_c = lc_ < -1 ? -1 : (lc_ > BLK ? BLK : (int)lc_);  // offsets > lim_c are masked
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = 32 * (kh * C::MTW + jj) + 16 * (i >> 3) + 8 * hf + (i & 7);
            if (off >= lim_n || off > lim_c) s[jj][i] = -INFINITY;
          }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[jj][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_tile = (mx == -INFINITY) ? -INFINITY : fmaf(mx, p.c, bias);
      if (__any(m_tile > m_run + kTau)) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        m_run = m_new;
      }
      const float nb = bias - (m_run == -INFINITY ? 0.f : m_run);

      // O^T += V^T P^T
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj) {
        const int j = kh * C::MTW + jj;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float pv[8];
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) pv[e8] = __builtin_amdgcn_exp2f(fmaf(s[jj][8 * s2 + e8], p.c, nb));
          l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
          const uint4 pk = make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                                      cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7]));
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            const int row = 32 * dt + ln;
            const int ch = (4 * j + 2 * s2 + hf) ^ swz<C::VCPR>(row);
            const uint4 a = *reinterpret_cast<const uint4 *>(vt + row * (BLK * 2) + ch * 16);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb, o[dt], 0, 0, 0);
          }
        }
      }
  };

  for (int c0 = e0; c0 < e1; c0 += C::LIST) {
    const int n = e1 - c0 < C::LIST ? e1 - c0 : C::LIST;
    for (int i = tid; i < n; i += C::NT) {
      lcol[i] = col[c0 + i];
      lbias[i] = lw ? lw[c0 + i] * kLog2e : 0.f;
    }
    __syncthreads();
    issue_tile(0, k0, v0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int i = 0; i < n; i += 2) {
      if (i + 1 < n) issue_tile(i + 1, k1, v1);
      compute_tile(i, k0, v0);
      __builtin_amdgcn_s_waitcnt(0);   // this wavefront's copies of tile i+1 have landed
      __syncthreads();                 // ... and everyone else's; stage 0 is free again
      if (i + 1 >= n) break;
      if (i + 2 < n) issue_tile(i + 2, k0, v0);
      compute_tile(i + 1, k1, v1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // merge the two key halves of every query group, normalise, store
  const float l_w = l_run + __shfl_xor(l_run, 32);
  // after the last barrier no tile is read any more: one buffer per query group
  float *scratch = reinterpret_cast<float *>(qg == 0 ? k0 : qg == 1 ? v0 : qg == 2 ? k1 : v1);
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
  const int64_t oi = (qi < N && sperm) ? (int64_t)sperm[bh * N + qi] : qi;
  if (qi < N && oi >= 0 && oi < N) {
    uint16_t *ob = out + b * p.os0 + h * p.os1 + oi * p.os2;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 o2 = *reinterpret_cast<const f32x4 *>(scratch + ((dt * 4 + i4) * 64 + lane) * 4);
        const float x0 = (o[dt][4 * i4] * a1 + o2[0] * a2) * inv;
        const float x1 = (o[dt][4 * i4 + 1] * a1 + o2[1] * a2) * inv;
        const float x2 = (o[dt][4 * i4 + 2] * a1 + o2[2] * a2) * inv;
        const float x3 = (o[dt][4 * i4 + 3] * a1 + o2[3] * a2) * inv;
        *reinterpret_cast<uint2 *>(ob + 32 * dt + 8 * i4 + 4 * hf) =
            make_uint2(cvt_pk_bf16(x0, x1), cvt_pk_bf16(x2, x3));
      }
    if (lse && hf == 0) lse[bh * N + oi] = l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int BLK, int D>
void launch_one(const AttnParams &p, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((attn_dimv_kernel<BLK, D>), dim3((unsigned)grid), dim3(DCfg<BLK, D>::NT), 0, s, p,
                     p.row_ptr, p.col, p.lw, p.order, p.sperm, p.o, p.lse);
}

}  // namespace

hipError_t launch_attn_dimv(const AttnParams &p, int block, int d, int64_t grid, hipStream_t s) {
  if (block == 128 && d == 128) launch_one<128, 128>(p, grid, s);
  else if (block == 128) launch_one<128, 64>(p, grid, s);
  else if (d == 128) launch_one<64, 128>(p, grid, s);
  else launch_one<64, 64>(p, grid, s);
  return hipGetLastError();
}

}  // namespace bsa
