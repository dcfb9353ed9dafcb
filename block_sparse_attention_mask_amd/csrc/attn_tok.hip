// Token-level attention over computational query sets for CDNA4 (gfx950).
//
// A computational query set (INTRA, section 3: a group of query tokens
// evaluated together, with a structured mapping to the key tokens it
// attends to) is given here by its query positions and its list of key
// positions; INTRA's Scatter and Gather maps and MC-Sparse's per-group token
// selection are all such lists.  For every query t of a set,
// o_t = sum_e softmax_e(q_t . k_{s_e} / sqrt(d)) v_{s_e} over the list
// entries e (InstaGen, section 3.1 Eq. (1)-(3)); entries outside the
// sequence and, when causal, keys s_e > t do not take part.  Outputs go back
// to the query positions (INTRA, section 4.8).
//
// Mapping to the hardware (one workgroup per set, or per run of the sets of
// 2 or 4 consecutive query heads of a KV group when their query slots and
// key lists are identical; head dim 128):
//   * Wavefront w owns 32 queries (query group, or head and query group) and
//     every key of every tile (one 32-key M tile per 32 keys of the tile), so
//     no merge is needed.
//   * 64-query sets of one head: 2 wavefronts over 32-key tiles, the list
//     staged 1024 entries at a time; 37 KB of LDS, so four sets run on a
//     CU at once, which hides more of each set's chain of dependent loads
//     (list, first gathers) than larger tiles would.
//   * 128-query sets (4 wavefronts) and runs of 2 or 4 heads' 64-query sets
//     (4 or 8 wavefronts): 64-key tiles, the list staged 2048 entries at a
//     time, two or one per CU.  With 2 or 4 heads every gathered tile serves
//     all of them, dividing the gather traffic per unit of work by 2 or 4.
//   * The sets are dealt to the XCDs in contiguous shares, so that an XCD
//     runs neighbouring sets, which list mostly the same keys, at the same
//     time and its L2 holds their K and V rows.
//   * The first chunk of a set's list is loaded into registers together with
//     its query slots; the normalised outputs are staged in LDS and written
//     as whole 256-byte rows.
//   * The selected K and V rows are gathered straight into LDS by
//     buffer_load_dwordx4 ... lds: each lane copies one 16-byte chunk of one
//     key row, with the row's position taken from the staged key list, so a
//     tile of arbitrary keys lands as two dense [key][dim] tiles.  Rows
//     past the list or outside the sequence read as zeros.
//   * S^T = K Q^T reads K chunks with ds_read_b128 (K rows are stored with
//     chunk c of row r at chunk position c ^ (r mod 16)).  O^T = V^T P^T needs
//     eight consecutive keys of one dim per lane: the V tile stays key-major
//     and two ds_read_b64_tr_b16 transpose reads per operand deliver them
//     (V rows are stored with chunk c of row r at c ^ (4 (r mod 4) +
//     2 ((r / 8) mod 2)), which spreads the eight rows and four chunks one
//     transpose read touches over all 64 banks).
//   * Tiles with keys that need the element mask (past the list, outside the
//     sequence, or after the set's first query when causal) are flagged
//     while the list is staged; only those tiles read key positions per
//     score.
//   * Software pipeline over two stages of K and of V: interval i computes
//     S(i+1) = K(i+1) Q^T in the same basic block as the exponentials of
//     S(i), then O += V(i) P(i), while the gathers of K(i+2) and V(i+1) are
//     in flight.
//   * Softmax in base 2, fp32; the running max is raised (and O rescaled)
//     only when a tile's max exceeds it by more than 8.
#include <type_traits>

#include "attn_common.h"

namespace bsa {
namespace tok {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int BQ, int HP, int BK_, int LIST_>
struct TCfg {
  static constexpr int D = 128;
  static constexpr int NQG = BQ / 32;             // query groups per head
  static constexpr int NW = HP * NQG;             // wavefronts: one per (head, query group)
  static constexpr int NT = 64 * NW;              // threads
  static constexpr int BK = BK_;                  // keys per tile
  static constexpr int MTW = BK / 32;             // 32-key M tiles per tile
  static constexpr int KS = D / 16;               // k-steps of K Q^T
  static constexpr int DT = D / 32;               // 32-dim M tiles of O^T
  static constexpr int TILE = BK * D * 2;         // bytes of a K or V tile
  static constexpr int NCOPY = TILE / 1024;       // 1 KB copies per tile (4 rows each)
  static constexpr int NC = NCOPY / NW;           // copies per wavefront per tile
  static constexpr int LIST = LIST_;              // list entries staged at a time
  static constexpr int NTL = LIST / BK;           // tiles per staged chunk
  static_assert(BK == 32 || BK == 64, "32- or 64-key tiles");
  static_assert(NCOPY % NW == 0, "whole copies per wavefront");
  static_assert(LIST % NT == 0 && NTL <= NT, "whole list entries per thread, one flag per thread");
  static_assert(NW * 8192 <= 4 * TILE, "every wavefront's output rows fit the stage buffers");
};

struct TokParams {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  float *lse;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  const int32_t *q_idx, *kv_ptr, *kv_idx;
  int64_t n_sets;   // B * Hq * sets per head
  int sets, Hq, G, N, causal;
  float c;          // softmax scale * log2(e)
};

__device__ __forceinline__ int vswz(int r) { return 4 * (r & 3) + 2 * ((r >> 3) & 1); }

template <int BQ, int HP, int BK_, int LIST_>
__device__ __forceinline__ void attn_tok_body(const TokParams &p) {
  using C = TCfg<BQ, HP, BK_, LIST_>;
  constexpr int D = C::D, MTW = C::MTW;
  // tile buffers K0, K1, V0, V1 (index 0-3), each C::TILE bytes
  __shared__ __attribute__((aligned(1024))) uint8_t stg[4][C::TILE];
  uint8_t *const k0 = stg[0], *const k1 = stg[1], *const v0 = stg[2], *const v1 = stg[3];
  __shared__ int32_t lcol[C::LIST];
  __shared__ int32_t tflag[C::NTL];
  __shared__ int32_t qmin_s;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < C::NW);
  const int ln = lane & 31, hf = lane >> 5;
  const int hd = wave / C::NQG, qg = wave % C::NQG;   // this wavefront's head of the run and query group
  // the set whose slots and list this workgroup reads: set i, or with two
  // heads the i-th set of an even head (its partner head's set is identical)
  // (set counts are below 2^31: 32-bit index arithmetic)
  // Workgroups are dispatched round-robin over the 8 XCDs; unit i (set, or
  // pair of sets) goes to the workgroup that makes XCD x run the x-th
  // contiguous share of the units, so that the sets an XCD runs at the same
  // time are neighbours, which list mostly the same keys, and its L2 holds
  // their K and V rows.
  const int nu = (int)gridDim.x, xcd = (int)(blockIdx.x & 7);
  const int i = xcd * (nu >> 3) + (xcd < (nu & 7) ? xcd : (nu & 7)) + (int)(blockIdx.x >> 3);
  int set0;
  if (HP == 1) {
    set0 = i;
  } else {
    const int pr = i / p.sets;
    set0 = (HP * pr) * p.sets + (i - pr * p.sets);
  }
  if (set0 >= p.n_sets) return;
  const int bh = set0 / p.sets + hd;   // this wavefront's head
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int g = h / p.G;
  const int N = p.N;
  const int e0 = p.kv_ptr[set0], e1 = p.kv_ptr[set0 + 1];
  // the first chunk of the list goes to registers at once: its loads then
  // overlap the query loads below instead of following them
  constexpr int PF = C::LIST / C::NT;
  int32_t pre[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int i = tid + C::NT * k;
    pre[k] = i < e1 - e0 ? p.kv_idx[e0 + i] : -1;
  }

  // this lane's query and, when causal, the set's first query (for the flags)
  const int32_t qraw = p.q_idx[(int64_t)set0 * BQ + qg * 32 + ln];
  const bool qok = qraw >= 0 && qraw < N;
  const int qi = qok ? qraw : -1;
  if (p.causal) {
    if (tid == 0) qmin_s = 0x7fffffff;
    __syncthreads();
    if (hd == 0 && qok) atomicMin(&qmin_s, qi);
  }

  const rsrc_t qrs = make_rsrc(p.q + b * p.qs0 + h * p.qs1, ((int64_t)(N - 1) * p.qs2 + D) * 2);
  const i32x4 krs = buffer_rsrc(p.k + b * p.ks0 + g * p.ks1, ((int64_t)(N - 1) * p.ks2 + D) * 2);
  const i32x4 vrs = buffer_rsrc(p.v + b * p.vs0 + g * p.vs1, ((int64_t)(N - 1) * p.vs2 + D) * 2);
  const uint32_t ks2b = (uint32_t)p.ks2 * 2, vs2b = (uint32_t)p.vs2 * 2;

  // Q^T fragment (B operand): lane (ln, hf) holds q[qi][16 ks + 8 hf .. +7]
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = qok ? (uint32_t)(((int64_t)qi * p.qs2 + ks * 16 + hf * 8) * 2) : kOOR;
    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  }

  // Copies: copy I (0..NCOPY-1) of a tile fills LDS bytes [1024 I, 1024 I + 1024)
  // of its stage, rows 4 I .. 4 I + 3; lane l writes row 4 I + l / 16 at chunk
  // position l % 16, which holds source chunk position ^ swizzle(row).  Tile
  // indices past the staged list read zeros.
  // Every copy's LDS address is this wavefront's base plus a compile-time
  // offset (buffer BUF, slot t).
  const int crow = lane >> 4, cpos = lane & 15;
  const uint32_t wbase =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)&stg[0][0] + (uint32_t)wave * 1024u;
  int n = 0;   // entries of the staged chunk
  auto issue = [&](int i, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;   // 0, 1: K buffers; 2, 3: V buffers
    static_for<0, C::NC>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      const int row = 4 * (wave + C::NW * t) + crow;
      const int li = i * C::BK + row;
      const int kp = li < n ? lcol[li] : -1;
      const bool ok = kp >= 0 && kp < N;
      if constexpr (BUF >= 2) {
        const uint32_t off = ok ? (uint32_t)kp * vs2b + ((cpos ^ vswz(row)) << 4) : kOOR;
        lds_copy16_at<(uint32_t)(BUF * C::TILE + 1024 * C::NW * t)>(vrs, wbase, off, 0u);
      } else {
        const uint32_t off = ok ? (uint32_t)kp * ks2b + ((cpos ^ (row & 15)) << 4) : kOOR;
        lds_copy16_at<(uint32_t)(BUF * C::TILE + 1024 * C::NW * t)>(krs, wbase, off, 0u);
      }
    });
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;

  // The keys of a tile: M tiles jj (32 keys each).  K
  // reads: the lane's score row of M tile t is key 32 t + key_of_row(ln);
  // chunk 2 ks + hf sits at (2 ks) ^ (hf ^ (key mod 16))
  int kbase[MTW], kx[MTW];
#pragma unroll
  for (int jj = 0; jj < MTW; ++jj) {
    const int kkey = 32 * jj + key_of_row(ln);
    kbase[jj] = kkey * (D * 2);
    kx[jj] = hf ^ (kkey & 15);
  }
  // V transpose reads: lane (gg = lane / 16, j = lane / 4 mod 4, qq = lane mod 4)
  // supplies the address of keys kb0 + 8 (gg / 2) + j (+4 for the second read),
  // dims 32 dt + 16 (gg mod 2) + 4 qq .. +3
  const int gg = lane >> 4, vj = (lane >> 2) & 3, qq = lane & 3;
  const int vrow0 = 8 * (gg >> 1) + vj;
  const int vcc = (2 * (gg & 1) + (qq >> 1)) ^ (2 * (gg >> 1));   // low two bits of the chunk position
  const int vhalf = (qq & 1) * 8;

  auto qk = [&](f32x16 (&s)[MTW], const uint8_t *kt) {
#pragma unroll
    for (int jj = 0; jj < MTW; ++jj)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[jj][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
      for (int jj = 0; jj < MTW; ++jj) {
        const uint4 a = *reinterpret_cast<const uint4 *>(kt + kbase[jj] + (((2 * ks) ^ kx[jj]) << 4));
        s[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[jj], 0, 0, 0);
      }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  f32x16 sa[MTW], sb[MTW];

  auto interval = [&](int i, f32x16 (&sc)[MTW], f32x16 (&sn)[MTW], const uint8_t *kt_next, const uint8_t *vt) {
    if (tflag[i]) {
      // element e of M tile t holds tile key 32 t + 8 hf + 16 (e >> 3) + (e & 7)
#pragma unroll
      for (int jj = 0; jj < MTW; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int li = i * C::BK + 32 * jj + 8 * hf + 16 * (e >> 3) + (e & 7);
          const int kp = li < n ? lcol[li] : -1;
          if (kp < 0 || kp >= N || (p.causal && kp > qi)) sc[jj][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < MTW; ++jj)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[jj][e]);
    mx = halves_max(mx);
    const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * p.c;
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
    const float nb = -(m_run == -INFINITY ? 0.f : m_run);
    bf16x8 pb[MTW][2];
    auto exps = [&]() {
#pragma unroll
      for (int jj = 0; jj < MTW; ++jj)
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
    // exponentials share one basic block; after the last tile it reads a
    // stage of zeros or a stale one and is never used
    qk(sn, kt_next);
    exps();
#pragma unroll
    for (int jj = 0; jj < MTW; ++jj)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int r0 = 32 * jj + 16 * s2 + vrow0;   // keys of the first transpose read
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const int pos = (4 * (dt ^ vj)) | vcc;
          const uint8_t *a0 = vt + r0 * (D * 2) + (pos << 4) + vhalf;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(a0));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(a0 + 4 * (D * 2)));
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[jj][s2], o[dt], 0, 0, 0);
        }
      }
  };

  // Staging of a list chunk of n entries: the tile flags start as "partial
  // last tile"; an entry outside the sequence or, when causal, after the
  // set's first query flags its tile.
  int qmin = 0;
  auto flags_init = [&]() {
    const int nt = (n + C::BK - 1) / C::BK;
    if (tid < C::NTL) tflag[tid] = (tid == nt - 1 && (n % C::BK)) ? 1 : 0;
  };
  auto put = [&](int i, int kp) {
    lcol[i] = kp;
    if (kp < 0 || kp >= N || (p.causal && kp > qmin)) atomicOr(&tflag[i / C::BK], 1);
  };
  // the first chunk from the registers, before the chunk loop, so that they
  // are free during it
  n = e1 - e0 < C::LIST ? e1 - e0 : C::LIST;
  flags_init();
  __syncthreads();
  if (p.causal) qmin = qmin_s;
#pragma unroll
  for (int k = 0; k < PF; ++k)
    if (tid + C::NT * k < n) put(tid + C::NT * k, pre[k]);
  for (int c0 = e0; c0 < e1; c0 += C::LIST) {
    n = e1 - c0 < C::LIST ? e1 - c0 : C::LIST;
    const int nt = (n + C::BK - 1) / C::BK;
    if (c0 != e0) {
      flags_init();
      __syncthreads();
      for (int i = tid; i < n; i += C::NT) put(i, p.kv_idx[c0 + i]);
    }
    __syncthreads();
    // prologue: K(0), V(0), K(1) resident, then S(0)
    issue(0, B0());
    issue(0, B2());
    if (nt > 1) issue(1, B1());
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    qk(sa, k0);
    // the first interval refills k0 with K(2): every wavefront must be done
    // reading K(0) first
    if (nt > 2) __syncthreads();
    for (int i = 0; i < nt; i += 2) {
      if (i + 2 < nt) issue(i + 2, B0());
      if (i + 1 < nt) issue(i + 1, B3());
      interval(i, sa, sb, k1, v0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (i + 1 >= nt) break;
      if (i + 3 < nt) issue(i + 3, B1());
      if (i + 2 < nt) issue(i + 2, B2());
      interval(i + 1, sb, sa, k0, v1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // normalise, store
  const float l_tot = halves_sum(l_run);
  const float m = m_run;
  // Normalised rows of this wavefront's 32 queries: staged in LDS as bf16
  // rows of 256 bytes (chunk c of row r at chunk position c ^ (r mod 16)),
  // then written out as whole rows, 16 lanes per row, instead of 16-byte
  // pieces of 32 rows per store (far fewer, full-line writes to drain
  // before the workgroup ends).  The stage buffers are free: every
  // wavefront is past the last tile.
  uint8_t *const obuf = &stg[0][0] + wave * 8192;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 x = {o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= inv;
      // dims 32 dt + 8 i4 + 4 hf .. +3: half hf of chunk 4 dt + i4 of row ln
      *reinterpret_cast<uint2 *>(obuf + ln * 256 + (((4 * dt + i4) ^ (ln & 15)) << 4) + 8 * hf) =
          make_uint2(cvt_pk_bf16(x[0], x[1]), cvt_pk_bf16(x[2], x[3]));
    }
  uint16_t *const obase = p.o + b * p.os0 + h * p.os1;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int row = 4 * t + (lane >> 4), ch = lane & 15;
    const int qr = __shfl(qi, row);   // lane `row` (hf = 0) holds that row's query
    const uint4 val = *reinterpret_cast<const uint4 *>(obuf + row * 256 + ((ch ^ (row & 15)) << 4));
    if (qr >= 0) *reinterpret_cast<uint4 *>(obase + (int64_t)qr * p.os2 + 8 * ch) = val;
  }
  if (p.lse && hf == 0 && qok) p.lse[(int64_t)bh * N + qi] = l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
}

// 64-query sets: 2 wavefronts over 32-key tiles, four per CU; 128-query
// sets and pairs of 64-query sets: 4 wavefronts over 64-key tiles, two per
// CU; runs of four 64-query sets: 8 wavefronts, one per CU
#define BSA_TOK_KERNEL(NAME, BQ, HP, BK, LIST)                                                       \
  __global__ __attribute__((amdgpu_flat_work_group_size(TCfg<BQ, HP, BK, LIST>::NT,                  \
                                                        TCfg<BQ, HP, BK, LIST>::NT),                 \
                            amdgpu_waves_per_eu(2, 2)))                                             \
  void NAME(const TokParams p) {                                                                   \
    attn_tok_body<BQ, HP, BK, LIST>(p);                                                             \
  }
BSA_TOK_KERNEL(attn_tok_64, 64, 1, 32, 1024)
BSA_TOK_KERNEL(attn_tok_128, 128, 1, 64, 2048)
BSA_TOK_KERNEL(attn_tok_64x2, 64, 2, 64, 2048)
BSA_TOK_KERNEL(attn_tok_64x4, 64, 4, 64, 2048)
#undef BSA_TOK_KERNEL

bool bad_strides(const int64_t s[3]) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || (s[i] & 7)) return true;
  return false;
}

}  // namespace tok
}  // namespace bsa

extern "C" int bsa_attn_tok_fwd(const bsa_tok_args *a, bsa_stream_t stream) {
  using namespace bsa;
  if (!a) return BSA_ERR_ARG;
  if (!a->q || !a->k || !a->v || !a->o || !a->q_idx || !a->kv_ptr) return BSA_ERR_ARG;
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->N <= 0 || a->n_sets < 0) return BSA_ERR_ARG;
  if (a->Hq % a->Hkv) return BSA_ERR_ARG;
  if (a->d != 128 || (a->set_size != 64 && a->set_size != 128)) return BSA_ERR_UNSUPPORTED;
  if (a->kv_share != 0 && a->kv_share != 2 && a->kv_share != 4) return BSA_ERR_ARG;
  if (a->kv_share && (a->set_size != 64 || (a->Hq / a->Hkv) % a->kv_share)) return BSA_ERR_UNSUPPORTED;
  if (!bsa_aligned16(a->q) || !bsa_aligned16(a->k) || !bsa_aligned16(a->v) || !bsa_aligned16(a->o))
    return BSA_ERR_ARG;
  if (tok::bad_strides(a->q_str) || tok::bad_strides(a->k_str) || tok::bad_strides(a->v_str) ||
      tok::bad_strides(a->o_str))
    return BSA_ERR_ARG;
  if (a->q_str[2] < a->d || a->k_str[2] < a->d || a->v_str[2] < a->d || a->o_str[2] < a->d) return BSA_ERR_ARG;
  if (a->o == a->q || a->o == a->k || a->o == a->v) return BSA_ERR_ARG;
  const int64_t lim = int64_t(1) << 30;
  if (((a->N - 1) * a->q_str[2] + a->d) * 2 >= lim || ((a->N - 1) * a->k_str[2] + a->d) * 2 >= lim ||
      ((a->N - 1) * a->v_str[2] + a->d) * 2 >= lim)
    return BSA_ERR_UNSUPPORTED;
  const int64_t n_sets = (int64_t)a->B * a->Hq * a->n_sets;
  if (n_sets >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  if (n_sets == 0) return BSA_OK;
  if (!a->kv_idx) return BSA_ERR_ARG;
  tok::TokParams p;
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = static_cast<const uint16_t *>(a->k);
  p.v = static_cast<const uint16_t *>(a->v);
  p.o = static_cast<uint16_t *>(a->o);
  p.lse = a->lse;
  p.qs0 = a->q_str[0]; p.qs1 = a->q_str[1]; p.qs2 = a->q_str[2];
  p.ks0 = a->k_str[0]; p.ks1 = a->k_str[1]; p.ks2 = a->k_str[2];
  p.vs0 = a->v_str[0]; p.vs1 = a->v_str[1]; p.vs2 = a->v_str[2];
  p.os0 = a->o_str[0]; p.os1 = a->o_str[1]; p.os2 = a->o_str[2];
  p.q_idx = a->q_idx;
  p.kv_ptr = a->kv_ptr;
  p.kv_idx = a->kv_idx;
  p.n_sets = n_sets;
  p.sets = a->n_sets;
  p.Hq = a->Hq;
  p.G = a->Hq / a->Hkv;
  p.N = (int)a->N;
  p.causal = a->causal ? 1 : 0;
  const float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->d);
  p.c = scale * kLog2e;
  hipStream_t s = bsa_hip_stream(stream);
  if (a->kv_share == 4) hipLaunchKernelGGL(tok::attn_tok_64x4, dim3((unsigned)(n_sets / 4)), dim3(512), 0, s, p);
  else if (a->kv_share == 2) hipLaunchKernelGGL(tok::attn_tok_64x2, dim3((unsigned)(n_sets / 2)), dim3(256), 0, s, p);
  else if (a->set_size == 64) hipLaunchKernelGGL(tok::attn_tok_64, dim3((unsigned)n_sets), dim3(128), 0, s, p);
  else hipLaunchKernelGGL(tok::attn_tok_128, dim3((unsigned)n_sets), dim3(256), 0, s, p);
  BSA_LAUNCH_CHECK();
  return BSA_OK;
}
