// Block-sparse softmax attention forward for a pair of query heads that share
// a KV head and list the same KV blocks (grouped-query attention with a
// pattern shared by the group's heads, as in the LLaMA-3.1-8B prefill of
// INTRA's Table 17: 32 query heads over 8 KV heads).  Semantics as in
// attn_pp.hip (InstaGen, section 3.1 Eq. (1)-(3) over the listed blocks, with
// the block's log-weight added to the scaled logit).
//
// Mapping (one workgroup of 8 wavefronts per pair of rows (b, h, u) and
// (b, h + 1, u), h even, both reading KV head g):
//   * Wavefront w owns the 32 queries of group w % 4 of head h + w / 4 and
//     walks every half tile (64 keys) of the row's blocks in order: half tile
//     j is keys 64 (j % 2) .. +63 of list entry j / 2.  One online softmax
//     per wavefront over all its keys, so no merge at the end.
//   * The two heads' wavefronts of a SIMD run half a tile apart, as the key
//     halves do in attn_pp.hip: head 0 runs M(0) E(0) M(1) ... M(T) in phases
//     0 .. 2T (T = 2 n half tiles), head 1 the same in phases 1 .. 2T + 1; in
//     every phase one wavefront of a SIMD issues MFMAs (M: O += V^T P^T of
//     half tile j - 1, then S = K Q^T of half tile j) while the other runs a
//     softmax step (E: mask, exponentials -> P of half tile j).
//   * Every staged half tile is read by both heads, one phase apart: K half
//     tile j in phases 2j and 2j + 1, V^T half tile j in phases 2j + 2 and
//     2j + 3.  So each phase stages one half tile (K in even phases, V^T in
//     odd ones), half of what a one-head workgroup stages per unit of work.
//     K(j) is copied in phase 2j - 4 into K buffer j % 3, V^T(j) in phase
//     2j - 1 into V^T buffer j % 3, and a buffer is refilled only after both
//     heads have read it.  The softmax step of the phase issues the copies
//     (head 1's E(j) copies K(j + 3), head 0's E(j) copies V^T(j + 1)); M
//     steps issue only LDS reads and MFMAs.  A wavefront waits, at the end of
//     each phase, for every copy it issued before its latest softmax step,
//     so a copy has landed by the end of the second phase after the one
//     that issued it (before phase 2j - 1 for K(j), first read in phase 2j;
//     before phase 2j + 2 for V^T(j), first read in phase 2j + 2).
//   * LDS layout, MFMA mapping, swizzle, list staging and the fixed-max
//     passes (a row whose probability total overflows 2^64 or stays below
//     2^-60 is recomputed from its cold tiles' max) are those of attn_pp.hip.
#include <type_traits>

#include "attn_pp_body.h"

namespace bsa {
namespace ppg {

template <int D>
struct GCfg {
  static constexpr int BLK = 128, HK = 64;          // block and half-tile keys
  static constexpr int NQG = 4, NW = 8, NT = 512;   // query groups, wavefronts, threads
  static constexpr int MTW = HK / 32;               // 32-key M tiles per half tile
  static constexpr int KS = D / 16;                 // k-steps of K Q^T
  static constexpr int DT = D / 32;                 // 32-dim M tiles of O^T
  static constexpr int KC = D / 8;                  // 16-byte chunks per K row
  static constexpr int VC = HK / 8;                 // 16-byte chunks per V^T half row
  static constexpr int NKC = HK * KC / 64;          // 1 KB copies per K half tile
  static constexpr int NVC = D * VC / 64;           // 1 KB copies per V^T half tile
  static constexpr int KB = NKC * 1024, VB = NVC * 1024;
  static constexpr int NSLOT = NKC / NQG;           // copies per softmax step (K or V^T)
  static constexpr int NM = MTW * (2 * DT + KS);    // MFMAs per matrix step
  static constexpr int LIST = 1024;                 // CSR entries staged in LDS at a time
  static_assert(NKC == NVC && KB == VB, "K and V^T half tiles have the same size");
  static_assert(NKC % NQG == 0, "whole copies per wavefront");
  static_assert((2 * MTW) % NSLOT == 0 || NSLOT % (2 * MTW) == 0, "copies spread evenly over the softmax step");
};

// LDS of one workgroup: K buffers 0-2, V^T buffers 3-5, each C::KB bytes at
// byte i * C::KB of smem; the staged list; the redo votes.
template <int D>
struct PgShared {
  alignas(1024) uint8_t smem[6 * GCfg<D>::KB];
  int32_t lcol[GCfg<D>::LIST];
  float lbias[GCfg<D>::LIST];
  int redo_vote[GCfg<D>::NW];
};

// Rows r0 and r1 (in [0, R), same batch and KV head, identical lists: the
// list of r0 is read), computed with the LDS arrays given: wavefronts 0-3
// serve r0, wavefronts 4-7 r1.
template <int D>
__device__ __forceinline__ void attn_ppg_body(const AttnParams &p, uint8_t *__restrict__ const smem,
                                              int32_t *__restrict__ const lcol, float *__restrict__ const lbias,
                                              int *__restrict__ const redo_vote, const int32_t r0, const int32_t r1,
                                              const int32_t *__restrict__ row_ptr,
                                              const int32_t *__restrict__ col, const float *__restrict__ lw,
                                              const int32_t *__restrict__ sperm, uint16_t *__restrict__ out,
                                              float *__restrict__ lse) {
  using C = GCfg<D>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < C::NW);
  const int ln = lane & 31, hf = lane >> 5;
  const int qg = wave % C::NQG, hd = wave / C::NQG;
  const int32_t rw = hd ? r1 : r0;   // this wavefront's row
  const int64_t bh = rw / p.nQB;
  const int u = (int)(rw - bh * p.nQB);
  const int64_t b = bh / p.Hq;
  const int h = (int)(bh - b * p.Hq);
  const int g = h / p.G;
  const int N = (int)p.N;
  const int e0 = row_ptr[r0], e1 = row_ptr[r0 + 1];
  const int nfull = N / C::BLK;
  const int mlim = p.causal ? (u < nfull ? u : nfull) : nfull;
  const int qi = u * C::BLK + qg * 32 + ln;   // this lane's query position

  const rsrc_t qrs = make_rsrc(p.q + b * p.qs0 + h * p.qs1, ((int64_t)(N - 1) * p.qs2 + D) * 2);
  const i32x4 krs = buffer_rsrc(p.k + b * p.ks0 + g * p.ks1, ((int64_t)(N - 1) * p.ks2 + D) * 2);
  const i32x4 vrs = buffer_rsrc(p.v + b * p.vs0 + g * p.vs1, (int64_t)D * p.vs2 * 2);
  const uint32_t ks2b = (uint32_t)p.ks2 * 2, vs2b = (uint32_t)p.vs2 * 2;

  const int qrow = (qi < N && p.gperm) ? p.gperm[bh * N + qi] : qi;
  const bool qok = qi < N && qrow >= 0 && qrow < N;
  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = qok ? (uint32_t)(((int64_t)qrow * p.qs2 + ks * 16 + hf * 8) * 2) : kOOR;
    qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  }

  // Copy slots of one half tile: slot t of the wavefront of query group qg
  // is copy c = qg + 4 t; copy c writes LDS bytes [1024 c, 1024 c + 1024) of
  // its buffer.  lok[t] / lov[t]: the lane's source offset within a K / V^T
  // half tile (source chunk position ^ swz(row), as in attn_pp.hip).
  uint32_t lok[C::NSLOT], lov[C::NSLOT];
#pragma unroll
  for (int t = 0; t < C::NSLOT; ++t) {
    const int c = qg + C::NQG * t;
    {
      const int s = c * 64 + lane, row = s / C::KC, ch = (s % C::KC) ^ swz<C::KC>(row);
      lok[t] = (uint32_t)row * ks2b + ch * 16;
    }
    {
      const int s = c * 64 + lane, row = s / C::VC, ch = (s % C::VC) ^ swz<C::VC>(row);
      lov[t] = (uint32_t)row * vs2b + ch * 16;
    }
  }
  const uint32_t wbase =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)smem + (uint32_t)qg * 1024u;

  int n = 0;   // entries of the current list chunk
  // list entry i (block index; 0 outside [0, n)), uniform over the wavefront
  auto entry = [&](int i) -> uint32_t {
    return __builtin_amdgcn_readfirstlane((uint32_t)lcol[(uint32_t)i < (uint32_t)n ? i : 0]);
  };
  // source byte offset of half tile j (block kb): K rows, or V^T key columns;
  // half tiles outside [0, 2n) read zeros (offsets past the buffer)
  auto ksrc = [&](int j, uint32_t kb) -> uint32_t {
    const uint32_t blk = kb < (uint32_t)p.nQB ? kb : 0u;
    return (uint32_t)j < (uint32_t)(2 * n) ? (blk * C::BLK + C::HK * (j & 1)) * ks2b : kOOR;
  };
  auto vsrc = [&](int j, uint32_t vb) -> uint32_t {
    const uint32_t blk = vb < (uint32_t)p.nQB ? vb : 0u;
    return (uint32_t)j < (uint32_t)(2 * n) ? (blk * C::BLK + C::HK * (j & 1)) * 2 : kOOR;
  };
  // copy slot T of a K half tile into K buffer BK / of a V^T half tile into
  // V^T buffer BV (buffer indices 0-2)
  auto copy_k = [&](auto tc, auto bkc, uint32_t base) {
    constexpr int T = decltype(tc)::value, BK = decltype(bkc)::value;
    lds_copy16_at<(uint32_t)(BK * C::KB + T * C::NQG * 1024)>(krs, wbase, lok[T] + base, 0u);
  };
  auto copy_v = [&](auto tc, auto bvc, uint32_t base) {
    constexpr int T = decltype(tc)::value, BV = decltype(bvc)::value;
    lds_copy16_at<(uint32_t)((3 + BV) * C::KB + T * C::NQG * 1024)>(vrs, wbase, lov[T] + base, 0u);
  };
  auto copy_k_all = [&](auto bkc, uint32_t base) {
    static_for<0, C::NSLOT>([&](auto tc) { copy_k(tc, bkc, base); });
  };
  auto copy_v_all = [&](auto bvc, uint32_t base) {
    static_for<0, C::NSLOT>([&](auto tc) { copy_v(tc, bvc, base); });
  };

  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // End of a phase: LDS reads done, every copy issued before this
  // wavefront's latest softmax step landed, then the barrier.
  auto end_phase = [&]() {
    __builtin_amdgcn_s_waitcnt(vm_lgkm0_wait_imm(C::NSLOT));
    barrier();
  };

  auto run = [&](auto hdc) {
    constexpr int HD = decltype(hdc)::value;
    float m_run = 0.f, l_run = 0.f, m_cold = -INFINITY;
    bool ovf = false;
    f32x16 o[C::DT];
    f32x16 s[C::MTW];
    bf16x8 pb[C::MTW][2];

    int ka[C::MTW];
#pragma unroll
    for (int jj = 0; jj < C::MTW; ++jj) {
      const int row = 32 * jj + key_of_row(ln);
      ka[jj] = row * C::KC * 16 + ((hf ^ swz<C::KC>(row)) << 4);
    }
    const int va = ln * C::VC * 16 + ((hf ^ swz<C::VC>(ln)) << 4);

    auto pin_results = [&]() {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) asm volatile("" ::"v"(o[dt]));
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj) {
        asm volatile("" ::"v"(s[jj]));
        asm volatile("" ::"v"(pb[jj][0]), "v"(pb[jj][1]));
      }
      asm volatile("" ::"v"(l_run));
    };

    // matrix step: O += V^T P^T (previous half tile), then S = K Q^T
    auto mstep = [&](const uint8_t *vt, const uint8_t *kt) {
      static_for<0, 2 * C::MTW * C::DT>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int jj = i / (2 * C::DT), s2 = (i / C::DT) % 2, dt = i % C::DT;
        const uint4 a = *reinterpret_cast<const uint4 *>(vt + ((va ^ (64 * jj + 32 * s2)) + 4096 * dt));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[jj][s2], o[dt], 0, 0, 0);
      });
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[jj][i] = 0.f;
      static_for<0, C::KS * C::MTW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        constexpr int ks = i / C::MTW, jj = i % C::MTW;
        const uint4 a = *reinterpret_cast<const uint4 *>(kt + (ka[jj] ^ (32 * ks)));
        s[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[jj], 0, 0, 0);
      });
      constexpr int kRA = 6;
      __builtin_amdgcn_sched_group_barrier(0x100, kRA, 0);
#pragma unroll
      for (int i = 0; i < C::NM - kRA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kRA, 0);
    };

    // what a softmax step E(j) reads from the list, read during M(j): its own
    // block and log-weight, and the block of the half tile it copies
    struct Pre {
      uint32_t eb, cb;
      float bias;
    };
    auto pre_of = [&](int j) -> Pre {
      Pre pr;
      pr.eb = entry(j >> 1);
      pr.cb = entry((HD == 0 ? j + 1 : j + 3) >> 1);
      pr.bias = __builtin_bit_cast(
          float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, lbias[(j >> 1) < n ? (j >> 1) : 0])));
      return pr;
    };

    // softmax step of half tile j: mask, exponentials -> pb, copies (head 0:
    // V^T(j+1) into V^T buffer CB, head 1: K(j+3) into K buffer CB) spread
    // over the groups of eight exponentials
    auto estep = [&](int j, auto cbc, const Pre &pr) {
      constexpr int CB = decltype(cbc)::value;
      const int ob = C::HK * (j & 1) + 8 * hf;   // key offset of this lane's first score row
      const uint32_t vb = pr.eb;
      const float bias = pr.bias;
      if (vb >= (uint32_t)mlim) {
        asm volatile("");   // keep this a branch: most tiles need no mask
        const int vbc = vb < (uint32_t)p.nQB ? (int)vb : p.nQB;
        const int kbase = vbc * C::BLK;
        const int lim_n = N - kbase > C::BLK ? C::BLK : (N - kbase < 0 ? 0 : N - kbase);
        const int lc = p.causal ? qi - kbase + 1 : C::BLK;
        const int lim1 = (lc < lim_n ? lc : lim_n) - ob - 1;
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t d = (uint32_t)(lim1 - (32 * jj + 16 * (e >> 3) + (e & 7)));
            s[jj][e] = fminf(s[jj][e], __uint_as_float((d & 0x80000000u) | 0x7f800000u));
          }
      }
      const uint32_t cbase = HD == 0 ? vsrc(j + 1, pr.cb) : ksrc(j + 3, pr.cb);
      const float nb = bias - m_run;
      float ls = 0.f;
      static_for<0, 2 * C::MTW>([&](auto gc) {
        constexpr int gi = decltype(gc)::value;
        constexpr int jj = gi / 2, s2 = gi % 2;
        float pv[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) pv[e8] = __builtin_amdgcn_exp2f(fmaf(s[jj][8 * s2 + e8], p.c, nb));
        ls += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        pb[jj][s2] = __builtin_bit_cast(bf16x8, make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                                                           cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7])));
        asm volatile("" ::"v"(pb[jj][s2]));
        static_for<gi * C::NSLOT / (2 * C::MTW), (gi + 1) * C::NSLOT / (2 * C::MTW)>([&](auto tc) {
          if constexpr (HD == 0) copy_v(tc, std::integral_constant<int, CB>(), cbase);
          else copy_k(tc, std::integral_constant<int, CB>(), cbase);
        });
      });
      const bool over = !(ls <= 0x1p64f);
      if (__any(over || ls < 0x1p-60f)) {
        float m = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = fmaxf(m, fmaf(s[jj][e], p.c, bias));
        m_cold = fmaxf(m_cold, halves_max(m));
        ovf = ovf || over;
      }
      l_run += ls;
    };

    // M(j) with K(j) in K buffer j % 3 and V^T(j - 1) in V^T buffer (j + 2) % 3;
    // E(j) copies into V^T buffer (j + 1) % 3 (head 0) or K buffer j % 3 (head 1)
    auto m_phase = [&](int j, auto kc) -> Pre {
      constexpr int K3 = decltype(kc)::value;   // j % 3
      // the matrix step issues ahead of the softmax step of the SIMD's other
      // wavefront: its MFMAs and operand reads are not held up behind VALU work
      __builtin_amdgcn_s_setprio(1);
      mstep(smem + (3 + (K3 + 2) % 3) * C::KB, smem + K3 * C::KB);
      __builtin_amdgcn_s_setprio(0);
      // the next softmax step's list reads come after every MFMA has issued:
      // their waits would otherwise hold up the first operand reads
      __builtin_amdgcn_sched_barrier(0);
      const Pre pr = pre_of(j);
      pin_results();
      end_phase();
      return pr;
    };
    auto e_phase = [&](int j, auto kc, const Pre &pr) {
      constexpr int K3 = decltype(kc)::value;
      estep(j, std::integral_constant<int, HD == 0 ? (K3 + 1) % 3 : K3>(), pr);
      pin_results();
      end_phase();
    };
    auto run_row = [&]() {
      const int T = 2 * n;
      if (HD == 1) {   // phase 0: head 1 idles and copies K(2) into K buffer 2
        copy_k_all(std::integral_constant<int, 2>(), ksrc(2, entry(1)));
        end_phase();
      }
#define BSA_PPG_STEP(K3)                                                \
  {                                                                     \
    const Pre pr = m_phase(j + K3, std::integral_constant<int, K3>()); \
    if (j + K3 == T) break;                                             \
    e_phase(j + K3, std::integral_constant<int, K3>(), pr);             \
  }
      for (int j = 0;; j += 3) {
        BSA_PPG_STEP(0)
        BSA_PPG_STEP(1)
        BSA_PPG_STEP(2)
      }
#undef BSA_PPG_STEP
      if (HD == 0) barrier();   // phase 2T + 1
    };

    for (int pass = 0;; ++pass) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
      l_run = 0.f;
      m_cold = -INFINITY;
      ovf = false;
      for (int c0 = e0; c0 < e1; c0 += C::LIST) {
        n = e1 - c0 < C::LIST ? e1 - c0 : C::LIST;
        for (int i = tid; i < n; i += C::NT) {
          lcol[i] = col[c0 + i];
          lbias[i] = lw ? lw[c0 + i] * kLog2e : 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj) pb[jj][0] = pb[jj][1] = bf16x8{};
        __syncthreads();
        // what the first phases read: K(0), K(1), V^T(0), and zeros for
        // "V^T(-1)" (V^T buffer 2); head 0's wavefronts copy K(0) and V^T(0),
        // head 1's K(1) and the zeros
        if (HD == 0) {
          copy_k_all(std::integral_constant<int, 0>(), ksrc(0, entry(0)));
          copy_v_all(std::integral_constant<int, 0>(), vsrc(0, entry(0)));
        } else {
          copy_k_all(std::integral_constant<int, 1>(), ksrc(1, entry(0)));
          copy_v_all(std::integral_constant<int, 2>(), kOOR);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        run_row();
        __builtin_amdgcn_s_waitcnt(0);   // every copy has landed before the buffers are reused
        __syncthreads();
      }
      if (pass > 0) break;
      const float lq = halves_sum(l_run);
      const bool over = halves_max(ovf ? 1.f : 0.f) > 0.f;
      const bool need = over || (lq < 0x1p-60f && m_cold > -INFINITY);
      if (lane == 0) redo_vote[wave] = __any(need) ? 1 : 0;
      __syncthreads();
      int any = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) any |= redo_vote[w];
      __syncthreads();
      if (!any) break;
      if (need) m_run = m_cold;
    }

    // normalise and store this wavefront's queries
    const float l_tot = halves_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    int oi = (qi < N && sperm) ? sperm[bh * N + qi] : qi;
    if (!(qi < N && oi >= 0 && oi < N)) oi = -1;   // padding query, or a scatter entry outside the rows
    // The rows are staged in this wavefront's 32 D bytes of the stage buffers
    // (every wavefront has passed the barrier after the last phase) as bf16
    // rows, chunk c of row r at chunk position c ^ (r mod KC), then written
    // out as whole rows, 64 / KC rows per store, instead of 16-byte pieces of
    // 32 rows (fewer, full-line writes to drain before the workgroup ends).
    static_assert(C::NW * 32 * 2 * D <= 6 * C::KB, "every wavefront's rows fit the stage buffers");
    uint8_t *const obuf = smem + wave * (32 * 2 * D);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float x0 = o[dt][4 * i4] * inv, x1 = o[dt][4 * i4 + 1] * inv;
        const float x2 = o[dt][4 * i4 + 2] * inv, x3 = o[dt][4 * i4 + 3] * inv;
        // dims 32 dt + 8 i4 + 4 hf .. +3: half hf of chunk 4 dt + i4 of row ln
        *reinterpret_cast<uint2 *>(obuf + ln * (2 * D) + (((4 * dt + i4) ^ (ln % C::KC)) << 4) + 8 * hf) =
            make_uint2(cvt_pk_bf16(x0, x1), cvt_pk_bf16(x2, x3));
      }
    uint16_t *const ob16 = out + b * p.os0 + h * p.os1;
    constexpr int RPS = 64 / C::KC;   // rows per store
#pragma unroll
    for (int t = 0; t < 32 / RPS; ++t) {
      const int row = RPS * t + lane / C::KC, ch = lane % C::KC;
      const int orow = __shfl(oi, row);   // lane `row` (hf = 0) holds that row's destination
      const uint4 val = *reinterpret_cast<const uint4 *>(obuf + row * (2 * D) + ((ch ^ (row % C::KC)) << 4));
      if (orow >= 0) *reinterpret_cast<uint4 *>(ob16 + (int64_t)orow * p.os2 + 8 * ch) = val;
    }
    if (lse && hf == 0 && oi >= 0) lse[bh * N + oi] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  };
  if (hd == 0) run(std::integral_constant<int, 0>());
  else run(std::integral_constant<int, 1>());
}

// Pairs of query heads: launch entry i serves the row of an even head (the
// launch table's entry, or pair-row i) and the same query block of the next
// head.  An entry outside the rows, or a row of an odd head, computes
// nothing.
#define BSA_PPG_KERNEL(NAME, D)                                                                      \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))     \
  void NAME(const AttnParams p, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col, \
            const float *__restrict__ lw, const int32_t *__restrict__ order,                         \
            const int32_t *__restrict__ sperm, uint16_t *__restrict__ out, float *__restrict__ lse) { \
    __shared__ PgShared<D> sh;                                                                      \
    int32_t r0;                                                                                     \
    if (order) {                                                                                    \
      r0 = order[blockIdx.x];                                                                       \
    } else {                                                                                        \
      const int64_t i = blockIdx.x, pr = i / p.nQB;                                                 \
      r0 = (int32_t)(2 * pr * p.nQB + (i - pr * p.nQB));                                           \
    }                                                                                               \
    if (r0 < 0 || r0 >= p.R) return;                                                                \
    if (((r0 / p.nQB) % p.Hq) & 1) return;                                                          \
    attn_ppg_body<D>(p, sh.smem, sh.lcol, sh.lbias, sh.redo_vote, r0, r0 + p.nQB, row_ptr, col, lw, sperm, \
                     out, lse);                                                                     \
  }
BSA_PPG_KERNEL(attn_ppg_128_128, 128)
BSA_PPG_KERNEL(attn_ppg_128_64, 64)
#undef BSA_PPG_KERNEL

// Rows and identical pairs in one launch: entry i serves row order[i] alone
// (the key-half body of attn_pp_body.h) or, when order2[i] is a row,
// together with row order2[i], which lists the same blocks (the pair body
// above; both bodies share one LDS allocation).  An entry outside the rows
// computes nothing.
template <int D>
union MixShared {
  pp::PpShared<D> one;
  PgShared<D> two;
};
#define BSA_PPX_KERNEL(NAME, D)                                                                      \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))     \
  void NAME(const AttnParams p, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col, \
            const float *__restrict__ lw, const int32_t *__restrict__ order,                         \
            const int32_t *__restrict__ order2, const int32_t *__restrict__ sperm,                  \
            uint16_t *__restrict__ out, float *__restrict__ lse) {                                  \
    __shared__ MixShared<D> sh;                                                                     \
    const int32_t r0 = order[blockIdx.x];                                                           \
    const int32_t r1 = order2[blockIdx.x];                                                          \
    if (r0 < 0 || r0 >= p.R) return;                                                                \
    if (r1 >= 0 && r1 < p.R)                                                                        \
      attn_ppg_body<D>(p, sh.two.smem, sh.two.lcol, sh.two.lbias, sh.two.redo_vote, r0, r1, row_ptr, col, \
                       lw, sperm, out, lse);                                                        \
    else                                                                                            \
      pp::attn_pp_body<D, false>(p, sh.one, r0, row_ptr, col, lw, sperm, out, lse);                 \
  }
BSA_PPX_KERNEL(attn_ppx_128_128, 128)
BSA_PPX_KERNEL(attn_ppx_128_64, 64)
#undef BSA_PPX_KERNEL

}  // namespace ppg

hipError_t launch_attn_ppx(const AttnParams &p, int d, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), t(512);
  if (d == 128)
    hipLaunchKernelGGL(ppg::attn_ppx_128_128, g, t, 0, s, p, p.row_ptr, p.col, p.lw, p.order, p.order2, p.sperm,
                       p.o, p.lse);
  else
    hipLaunchKernelGGL(ppg::attn_ppx_128_64, g, t, 0, s, p, p.row_ptr, p.col, p.lw, p.order, p.order2, p.sperm,
                       p.o, p.lse);
  return hipGetLastError();
}

hipError_t launch_attn_ppg(const AttnParams &p, int d, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), t(512);
  if (d == 128)
    hipLaunchKernelGGL(ppg::attn_ppg_128_128, g, t, 0, s, p, p.row_ptr, p.col, p.lw, p.order, p.sperm, p.o, p.lse);
  else
    hipLaunchKernelGGL(ppg::attn_ppg_128_64, g, t, 0, s, p, p.row_ptr, p.col, p.lw, p.order, p.sperm, p.o, p.lse);
  return hipGetLastError();
}

}  // namespace bsa
