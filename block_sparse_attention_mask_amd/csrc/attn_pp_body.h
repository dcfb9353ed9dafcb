// Block-sparse softmax attention forward for CDNA4 (gfx950): 128-query
// blocks, V dim-major, ping-pong schedule.
//
// Semantics as in InstaGen, section 3.1 Eq. (1)-(3) with the listed block's
// additive log-weight (Algorithm 1): for every query t of query block u,
// o_t = sum_s softmax_s(q_t.k_s / sqrt(d) + log w_v(s)) v_s over the keys of
// the KV blocks listed in row (b, h, u).  Keys past N and, when causal,
// keys s > t do not take part.
//
// Mapping to the hardware (one workgroup of 8 wavefronts per CSR row):
//   * Wavefront w owns the 32 queries of group w % 4 and the key half w / 4
//     (keys 0-63 or 64-127 of every 128-key tile).  The two halves keep
//     separate online-softmax states, merged once through LDS at the end.
//     Wavefronts w and w + 4 share a SIMD.
//   * The two halves run half a tile apart.  Time is cut into phases ended by
//     workgroup barriers; in each phase one wavefront of a SIMD runs its
//     matrix step (O += V^T P^T for its previous tile, then S = K Q^T for its
//     next one: 32 MFMAs fed from LDS) while the other runs the softmax of its
//     current tile (mask, max, exponentials: vector ALU only), so the matrix
//     cores and the vector ALUs of a SIMD work at the same time.  Half 0 does
//     its matrix steps in even phases, half 1 in odd phases.
//   * A half tile (64 keys of K, or V^T for 64 keys) is read in exactly one
//     phase by the four wavefronts of its half and lives in one of two LDS
//     buffers of its kind.  At the start of phase f the buffers read in phase
//     f-1 are refilled, by buffer_load ... lds copies, with the half tiles
//     read in phase f+2, so every copy has three phases to land.  All eight
//     wavefronts take part: each issues the same number of 1 KB copies per
//     phase, spread between its MFMAs or exponentials so that the vector
//     memory queue never holds up a whole step.  A wait for all but the last
//     two phases' copies, then the barrier, publishes the half tiles of the
//     next phase.  Entries past the end of the list are copied from offsets
//     past the buffer (zeros), which keeps the per-phase counts fixed.
//   * LDS rows are not padded: the 16-byte chunk c of row r is stored at
//     chunk position c ^ f(r) (f(r) = r mod 16 for 16-chunk rows, (r / 2)
//     mod 8 for 8-chunk rows), so the 16 lanes that read 16 different rows in
//     one 16-byte read hit 16 different bank groups.  The copies apply the
//     permutation on the source side; a reader forms each address with one
//     XOR.  S^T = K Q^T and O^T = V^T P^T use v_mfma_f32_32x32x16_bf16 with the
//     row-to-key map of key_of_row, so the eight probabilities a lane holds
//     per PV k-step are eight consecutive keys and the V^T operand is one
//     16-byte read.
//   * Softmax in base 2, fp32, p = 2^(c s + lw - m) with c = log2(e)/sqrt(d).
//     No per-tile max is taken: the running max m (starting at 0) is moved,
//     O and l rescaled and the tile's exponentials redone, only when a
//     lane's 32 probabilities of the tile sum past 32 * 2^8 (so some
//     probability exceeded 2^8), or while the lane's sum so far is below
//     2^-64 (nothing accumulated, or only underflowing probabilities).
//   * The row's list is staged in LDS, up to 1024 entries at a time: copied
//     from the CSR column array, or walked out of the row's CRM words
//     (ScalingAttention, section 7.3) with each wavefront taking a 4-bit
//     slice of every word.
//   * K tile offsets go into the range-checked lane offset, so rows at or
//     past N of a partial last block read as zeros; V^T rows hold every key
//     of every block, so their tile offset is scalar.
#pragma once
#include <type_traits>

#include "attn_common.h"

namespace bsa {
namespace pp {

template <int D>
struct PCfg {
  static constexpr int BLK = 128, HK = 64;          // block and half-tile keys
  static constexpr int NQG = 4, NW = 8, NT = 512;   // query groups, wavefronts, threads
  static constexpr int MTW = HK / 32;               // 32-key M tiles per half
  static constexpr int KS = D / 16;                 // k-steps of K Q^T
  static constexpr int DT = D / 32;                 // 32-dim M tiles of O^T
  static constexpr int KC = D / 8;                  // 16-byte chunks per K row
  static constexpr int VC = HK / 8;                 // 16-byte chunks per V^T half row
  static constexpr int NKC = HK * KC / 64;          // 1 KB copies per K half tile
  static constexpr int NVC = D * VC / 64;           // 1 KB copies per V^T half tile
  // the four softmax-step wavefronts of a phase issue all of its copies
  static constexpr int NSK = NKC / NQG, NSV = NVC / NQG;
  static constexpr int NSLOT = NSK + NSV;           // copies per softmax step
  static constexpr int KB = NKC * 1024, VB = NVC * 1024;
  static constexpr int NM = MTW * (2 * DT + KS);    // MFMAs per matrix step
  static constexpr int LIST = 1024;                 // CSR entries staged in LDS at a time
  static_assert(NKC % NQG == 0 && NVC % NQG == 0, "whole copies per wavefront");
  static_assert((2 * MTW) % NSLOT == 0 || NSLOT % (2 * MTW) == 0, "copies spread evenly over the softmax step");
  static_assert(64 * DT * 16 * 4 <= KB, "merge data of a query group fits a K buffer");
};

// LDS of one workgroup: K buffers 0-3 (kx0, kx1, ky0, ky1), V^T buffers 4-7
// (vx0, vx1, vy0, vy1), each C::KB bytes (buffer i at byte i * C::KB of
// smem); the staged list; per key half and query group the merge values (l,
// cold-tile max, overflow flag, running max); the redo votes.
template <int D>
struct PpShared {
  alignas(1024) uint8_t smem[8 * PCfg<D>::KB];
  int32_t lcol[PCfg<D>::LIST];
  float lbias[PCfg<D>::LIST];
  float mrg[2][4][PCfg<D>::NQG][64];
  int redo_vote[PCfg<D>::NW];
};

// Row r (in [0, R)) of the workgroup, computed with the LDS in sh.
template <int D, bool kCrm>
__device__ __forceinline__ void attn_pp_body(const AttnParams &p, PpShared<D> &sh, const int32_t r,
                                             const int32_t *__restrict__ row_ptr,
                                             const int32_t *__restrict__ col, const float *__restrict__ lw,
                                             const int32_t *__restrict__ sperm, uint16_t *__restrict__ out,
                                             float *__restrict__ lse) {
  using C = PCfg<D>;
  static_assert(C::KB == C::VB, "K and V^T half tiles have the same size");
  constexpr int KX0 = 0, KX1 = 1, KY0 = 2, KY1 = 3, VX0 = 4, VX1 = 5, VY0 = 6, VY1 = 7;
  // the arrays of sh do not overlap
  uint8_t *__restrict__ const smem = sh.smem;
  int32_t *__restrict__ const lcol = sh.lcol;
  float *__restrict__ const lbias = sh.lbias;
  auto &mrg = sh.mrg;
  int *__restrict__ const redo_vote = sh.redo_vote;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < C::NW);
  const int ln = lane & 31, hf = lane >> 5;
  const int qg = wave % C::NQG, kh = wave / C::NQG;
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
  const int nfull = N / C::BLK;
  const int mlim = p.causal ? (u < nfull ? u : nfull) : nfull;
  const int qi = u * C::BLK + qg * 32 + ln;   // this lane's query position

  const rsrc_t qrs = make_rsrc(p.q + b * p.qs0 + h * p.qs1, ((int64_t)(N - 1) * p.qs2 + D) * 2);
  const i32x4 krs = buffer_rsrc(p.k + b * p.ks0 + g * p.ks1, ((int64_t)(N - 1) * p.ks2 + D) * 2);
  const i32x4 vrs = buffer_rsrc(p.v + b * p.vs0 + g * p.vs1, (int64_t)D * p.vs2 * 2);
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

  // Copy slots.  Slot t of the wavefront of query group qg is copy
  // c = qg + 4 t of a pair of half tiles: K copy c for t < NSK, else V^T copy
  // c - NKC.  Copy c writes LDS bytes [1024 c, 1024 c + 1024) of its buffer;
  // lane l writes LDS slot 64 c + l, which holds (row, chunk position) =
  // divmod(slot, row chunks), so the lane reads source chunk position ^
  // swz(row).  lo[t] is that source offset within the half tile.
  uint32_t lo[C::NSLOT];
#pragma unroll
  for (int t = 0; t < C::NSLOT; ++t) {
    const int c = qg + C::NQG * t;
    if (t < C::NSK) {
      const int s = c * 64 + lane, row = s / C::KC, ch = (s % C::KC) ^ swz<C::KC>(row);
      lo[t] = (uint32_t)row * ks2b + ch * 16;
    } else {
      const int s = (c - C::NKC) * 64 + lane, row = s / C::VC, ch = (s % C::VC) ^ swz<C::VC>(row);
      lo[t] = (uint32_t)row * vs2b + ch * 16;
    }
  }
  // LDS address of this wavefront's first copy destination (buffer 0, copy
  // c = qg); every copy's M0 is this plus a compile-time offset
  const uint32_t wbase =
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)smem + (uint32_t)qg * 1024u;

  int n = 0;   // entries of the current list chunk
  // Source offsets of a phase's half tiles: K entry ki and V^T entry vi of
  // half hh.  Entries outside [0, n) read zeros (offsets past the buffer).
  struct Src {
    uint32_t kbase, vso, vadd;
  };
  // list entry i (block index; 0 outside [0, n)), uniform over the wavefront
  auto entry = [&](int i) -> uint32_t {
    return __builtin_amdgcn_readfirstlane((uint32_t)lcol[(uint32_t)i < (uint32_t)n ? i : 0]);
  };
  auto src_from = [&](int hh, int ki, int vi, uint32_t kb, uint32_t vb) -> Src {
    const bool kin = (uint32_t)ki < (uint32_t)n, vin = (uint32_t)vi < (uint32_t)n;
    const uint32_t kblk = kb < (uint32_t)p.nQB ? kb : 0u;
    const uint32_t vblk = vb < (uint32_t)p.nQB ? vb : 0u;
    Src sr;
    sr.kbase = kin ? (kblk * C::BLK + C::HK * hh) * ks2b : kOOR;
    sr.vso = vin ? (vblk * C::BLK + C::HK * hh) * 2 : 0u;
    sr.vadd = vin ? 0u : kOOR;
    return sr;
  };
  auto src_of = [&](int hh, int ki, int vi) -> Src { return src_from(hh, ki, vi, entry(ki), entry(vi)); };
  // What a softmax step reads from the staged list: its copy sources (K entry
  // j+2, V^T entry j+1) and its own block and log-weight.  Read one phase
  // ahead, during the same wavefront's matrix step, so that the softmax step
  // does not start with an LDS wait behind the matrix steps' operand reads.
  struct Pre {
    uint32_t kb, vb, eb;
    float bias;
  };
  auto pre_of = [&](int j) -> Pre {
    Pre pr;
    pr.kb = entry(j + 2);
    pr.vb = entry(j + 1);
    pr.eb = entry(j);
    pr.bias = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, lbias[j < n ? j : 0])));
    return pr;
  };
  // copy slot T of a phase into K buffer BK or V^T buffer BV
  auto copy_slot = [&](auto tc, auto bkc, auto bvc, const Src &sr) {
    constexpr int T = decltype(tc)::value, BK = decltype(bkc)::value, BV = decltype(bvc)::value;
    if constexpr (T < C::NSK)
      lds_copy16_at<(uint32_t)(BK * C::KB + T * C::NQG * 1024)>(krs, wbase, lo[T] + sr.kbase, 0u);
    else
      lds_copy16_at<(uint32_t)(BV * C::KB + (T - C::NSK) * C::NQG * 1024)>(vrs, wbase, lo[T] + sr.vadd, sr.vso);
  };
  auto copy_all = [&](auto bkc, auto bvc, const Src &sr) {
    static_for<0, C::NSLOT>([&](auto tc) { copy_slot(tc, bkc, bvc, sr); });
  };

  // End of a phase: this wavefront's LDS reads are done and every copy it
  // issued before its latest softmax step (two phases ago at the latest) has
  // landed; then the barrier.  The empty asm statements keep the compiler
  // from moving memory accesses across the barrier.
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto end_phase = [&]() {
    __builtin_amdgcn_s_waitcnt(vm_lgkm0_wait_imm(C::NSLOT));
    barrier();
  };

  // Everything from here on is instantiated per key half (KH = kh), so that
  // each half's accumulators live in one set of registers and every LDS
  // buffer a step touches is a known object.
  auto half = [&](auto khc) {
    constexpr int KH = decltype(khc)::value;
    // Online-softmax state of this lane's query over its key half.  The
    // running max m_run stays fixed for a whole pass (0 in the first), so O
    // is only ever written by the MFMAs.  A tile whose probabilities sum past
    // 2^64, or below 2^-60, is "cold": its max is folded into m_cold (and an
    // overflow is remembered).  A row that overflowed, or whose total stays
    // below 2^-60, is computed again from m_cold (second pass).
    float m_run = 0.f, l_run = 0.f, m_cold = -INFINITY;
    bool ovf = false;
    f32x16 o[C::DT];
    f32x16 s[C::MTW];
    bf16x8 pb[C::MTW][2];

    // LDS read addresses: K operand (jj, ks) at ka[jj] ^ 32 ks, V^T operand
    // (jj, s2, dt) at (va ^ (64 jj + 32 s2)) + 4096 dt
    int ka[C::MTW];
#pragma unroll
    for (int jj = 0; jj < C::MTW; ++jj) {
      const int row = 32 * jj + key_of_row(ln);
      ka[jj] = row * C::KC * 16 + ((hf ^ swz<C::KC>(row)) << 4);
    }
    const int va = ln * C::VC * 16 + ((hf ^ swz<C::VC>(ln)) << 4);
    const int ob = C::HK * KH + 8 * hf;   // key offset of this lane's first score row

    // The steps of one phase must run in that phase: register-only work (MFMAs,
    // exponentials) could otherwise be moved by the compiler across the
    // barrier into the neighbouring phase, where the SIMD's other wavefront
    // does the same kind of work.  An empty asm statement that uses every
    // result handed to the next phase pins it.
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

    // Matrix step: O += V^T P^T (previous tile), then S = K Q^T (this tile);
    // one 16-byte LDS read per MFMA.  Before the first tile pb is zero and
    // the V^T buffer holds zeros; after the last one S is not used.
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
      // keep kRA operand reads in flight ahead of the MFMAs
      constexpr int kRA = 6;
      __builtin_amdgcn_sched_group_barrier(0x100, kRA, 0);
#pragma unroll
      for (int i = 0; i < C::NM - kRA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, kRA, 0);
    };

    // softmax step of list entry i: mask, exponentials against the fixed
    // running max -> pb, with the phase's copies spread over the four groups
    // of eight exponentials; cold tiles fold their max into m_cold
    auto estep = [&](const Pre &pr, auto bkc, auto bvc, const Src &sr) {
      const uint32_t vb = pr.eb;
      const float bias = pr.bias;
      if (vb >= (uint32_t)mlim) {
        asm volatile("");   // keep this a branch: most tiles need no mask
        // keys past N (last block) and, when causal, keys after the query; a
        // block index outside the rows masks every key.  Element e of M tile
        // jj holds key offset ob + 32 jj + 16 (e >> 3) + (e & 7) in the block;
        // offsets above lim1 (relative to ob) are masked by a min with -inf,
        // formed from the sign of lim1 - offset (no per-element lane masks).
        const int vbc = vb < (uint32_t)p.nQB ? (int)vb : p.nQB;
        const int kbase = vbc * C::BLK;
        const int lim_n = N - kbase > C::BLK ? C::BLK : (N - kbase < 0 ? 0 : N - kbase);   // offsets >= lim_n: padding
        const int lc = p.causal ? qi - kbase + 1 : C::BLK;                                  // offsets >= lc: after the query
        const int lim1 = (lc < lim_n ? lc : lim_n) - ob - 1;
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t d = (uint32_t)(lim1 - (32 * jj + 16 * (e >> 3) + (e & 7)));
            s[jj][e] = fminf(s[jj][e], __uint_as_float((d & 0x80000000u) | 0x7f800000u));
          }
      }
      const float nb = bias - m_run;
      float ls = 0.f;
      static_for<0, 2 * C::MTW>([&](auto gc) {
        constexpr int gi = decltype(gc)::value;   // exponential group; its copies follow it
        constexpr int jj = gi / 2, s2 = gi % 2;
        float pv[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) pv[e8] = __builtin_amdgcn_exp2f(fmaf(s[jj][8 * s2 + e8], p.c, nb));
        ls += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        pb[jj][s2] = __builtin_bit_cast(bf16x8, make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                                                           cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7])));
        asm volatile("" ::"v"(pb[jj][s2]));
        static_for<gi * C::NSLOT / (2 * C::MTW), (gi + 1) * C::NSLOT / (2 * C::MTW)>(
            [&](auto tc) { copy_slot(tc, bkc, bvc, sr); });
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

    // Phase loop.  Half 0 runs M(0) E(0) M(1) ... E(n-1) M(n) in phases
    // 0 .. 2n and idles in phase 2n+1; half 1 idles in phase 0 and runs the
    // same steps in phases 1 .. 2n+1.  M(j) reads V^T entry j-1 of this half
    // from vmine[(j-1) & 1] and K entry j from kmine[j & 1].  The copies of
    // phase f are those of half (f odd ? 0 : 1), K entry (f+3)/2 into that
    // half's K buffer (entry & 1), V^T entry (f+1)/2 into its V^T buffer
    // (entry & 1), and that half runs the phase's softmax step (in phase 0,
    // where half 1 idles, it only copies): only softmax steps copy, so the
    // matrix steps issue nothing but LDS reads and MFMAs.  In phase 2n+1
    // nothing is copied (entries past the list, never read).
    constexpr int KM0 = KH ? KY0 : KX0, KM1 = KH ? KY1 : KX1;
    constexpr int VM0 = KH ? VY0 : VX0, VM1 = KH ? VY1 : VX1;
    auto m_phase = [&](int j, auto par) -> Pre {
      constexpr int P = decltype(par)::value;   // j & 1
      // the matrix step issues ahead of the softmax step of the SIMD's other
      // wavefront: its MFMAs and operand reads are not held up behind VALU work
      __builtin_amdgcn_s_setprio(1);
      mstep(smem + (P ? VM0 : VM1) * C::KB, smem + (P ? KM1 : KM0) * C::KB);
      __builtin_amdgcn_s_setprio(0);
      // the next softmax step's list reads come after every MFMA has issued:
      // their waits would otherwise hold up the first operand reads
      __builtin_amdgcn_sched_barrier(0);
      const Pre pr = pre_of(j);
      pin_results();
      end_phase();
      return pr;
    };
    auto e_phase = [&](int j, auto par, const Pre &pr) {
      constexpr int P = decltype(par)::value;
      // phase 2j+1+KH: this half, K entry j+2 into kmine[j & 1], V^T entry
      // j+1 into vmine[(j+1) & 1]
      const Src sr = src_from(KH, j + 2, j + 1, pr.kb, pr.vb);
      estep(pr, std::integral_constant<int, P ? KM1 : KM0>(), std::integral_constant<int, P ? VM0 : VM1>(), sr);
      pin_results();
      end_phase();
    };
    auto run_half = [&]() {
      using Z = std::integral_constant<int, 0>;
      using O = std::integral_constant<int, 1>;
      if (KH == 1) {   // phase 0: half 1, K entry 1 into ky1, V^T entry 0 into vy0
        const Src sr = src_of(1, 1, 0);
        copy_all(std::integral_constant<int, KY1>(), std::integral_constant<int, VY0>(), sr);
        end_phase();
      }
      for (int j = 0;; j += 2) {
        const Pre p0 = m_phase(j, Z());
        if (j == n) break;
        e_phase(j, Z(), p0);
        const Pre p1 = m_phase(j + 1, O());
        if (j + 1 == n) break;
        e_phase(j + 1, O(), p1);
      }
      if (KH == 0) barrier();   // phase 2n+1
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
        if constexpr (kCrm) {
          if (c0 > 0 || pass > 0) bsa_crm_walk(crow, p.crm_words, p.crm_tail, c0, n, lcol, wave, C::NW, lane);
          for (int i = tid; i < n; i += C::NT) lbias[i] = 0.f;
        } else {
          // the list arguments are read again from the argument block here,
          // so that they hold no scalar registers during the phase loop
          const kparams_t pk = kernel_params();
          const int32_t *const col_c = pk->col;
          const float *const lw_c = pk->lw;
          for (int i = tid; i < n; i += C::NT) {
            lcol[i] = col_c[c0 + i];
            lbias[i] = lw_c ? lw_c[c0 + i] * kLog2e : 0.f;
          }
        }
        // the first matrix step multiplies pb by the zero "V^T entry -1"
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj) pb[jj][0] = pb[jj][1] = bf16x8{};
        __syncthreads();
        // what the first phases read: K entries 0 and 1 and V^T entry 0 of half
        // 0, K entry 0 of half 1, and zeros for "V^T entry -1" of both halves
        // (each wavefront copies its query group's slots of one or two sets)
        if (KH == 0) {
          copy_all(std::integral_constant<int, KX0>(), std::integral_constant<int, VX0>(), src_of(0, 0, 0));
          copy_all(std::integral_constant<int, KY0>(), std::integral_constant<int, VY1>(), src_of(1, 0, -1));
        } else {
          copy_all(std::integral_constant<int, KX1>(), std::integral_constant<int, VX1>(), src_of(0, 1, -1));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        run_half();
        __builtin_amdgcn_s_waitcnt(0);   // every copy has landed before the buffers are reused
        __syncthreads();
      }
      // per query (both lanes of it): l over this key half, cold max, overflow
      const float lq = halves_sum(l_run);
      mrg[KH][0][qg][lane] = lq;
      mrg[KH][1][qg][lane] = m_cold;
      mrg[KH][2][qg][lane] = halves_max(ovf ? 1.f : 0.f);
      mrg[KH][3][qg][lane] = m_run;
      __syncthreads();
      if (pass > 0) break;
      const float mc = fmaxf(mrg[0][1][qg][lane], mrg[1][1][qg][lane]);
      const bool over = mrg[0][2][qg][lane] + mrg[1][2][qg][lane] > 0.f;
      const bool need = over || (mrg[0][0][qg][lane] + mrg[1][0][qg][lane] < 0x1p-60f && mc > -INFINITY);
      const bool wneed = __any(need);
      if (lane == 0) redo_vote[wave] = wneed ? 1 : 0;
      __syncthreads();
      int any = 0;
#pragma unroll
      for (int w = 0; w < C::NW; ++w) any |= redo_vote[w];
      __syncthreads();   // votes and merge values are read before they are written again
      if (!any) break;
      if (need) m_run = mc;   // both halves of the query start from the same max
    }

    // merge the two key halves of every query group, normalise, store
    float *scratch = reinterpret_cast<float *>(smem + qg * C::KB);
    if (KH == 1) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<f32x4 *>(scratch + ((dt * 4 + i4) * 64 + lane) * 4) =
              f32x4{o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
    }
    __syncthreads();
    if (KH != 0) return;
    const float l_w = mrg[0][0][qg][lane];
    const float m2 = mrg[1][3][qg][lane];
    const float l2 = mrg[1][0][qg][lane];
    // A half with nothing accumulated (l = 0) takes no part, whatever running
    // max it holds: its max may sit far above the other half's, and a weight
    // 2^(m_other - m) would then underflow.
    const float m = l_w > 0.f ? (l2 > 0.f ? fmaxf(m_run, m2) : m_run) : m2;
    const float a1 = l_w > 0.f ? __builtin_amdgcn_exp2f(m_run - m) : 0.f;
    const float a2 = l2 > 0.f ? __builtin_amdgcn_exp2f(m2 - m) : 0.f;
    const float l_tot = l_w * a1 + l2 * a2;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    // the output arguments are read again here from the kernel's argument
    // block (through a pointer the compiler cannot follow), so that none of
    // them occupies a scalar register during the phase loop
    const kparams_t pk = kernel_params();
    const int32_t *const sperm_e = pk->sperm;
    int oi = (qi < N && sperm_e) ? sperm_e[bh * N + qi] : qi;
    if (!(qi < N && oi >= 0 && oi < N)) oi = -1;   // padding query, or a scatter entry outside the rows
    // Normalised rows of this wavefront's 32 queries: staged in its V^T buffer
    // (free once the last phase has passed) as bf16 rows of 2 D bytes, chunk c
    // of row r at chunk position c ^ (r mod KC), then written out as whole
    // rows, 64 / KC rows per store, instead of 16-byte pieces of 32 rows
    // (fewer, full-line writes to drain before the workgroup ends).
    uint8_t *const obuf = smem + (VX0 + qg) * C::KB;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 o2 = *reinterpret_cast<const f32x4 *>(scratch + ((dt * 4 + i4) * 64 + lane) * 4);
        const float x0 = (o[dt][4 * i4] * a1 + o2[0] * a2) * inv;
        const float x1 = (o[dt][4 * i4 + 1] * a1 + o2[1] * a2) * inv;
        const float x2 = (o[dt][4 * i4 + 2] * a1 + o2[2] * a2) * inv;
        const float x3 = (o[dt][4 * i4 + 3] * a1 + o2[3] * a2) * inv;
        // dims 32 dt + 8 i4 + 4 hf .. +3: half hf of chunk 4 dt + i4 of row ln
        *reinterpret_cast<uint2 *>(obuf + ln * (2 * D) + (((4 * dt + i4) ^ (ln % C::KC)) << 4) + 8 * hf) =
            make_uint2(cvt_pk_bf16(x0, x1), cvt_pk_bf16(x2, x3));
      }
    uint16_t *const ob16 = pk->o + b * pk->os0 + h * pk->os1;
    const int64_t os2 = pk->os2;
    float *const lse_e = pk->lse;
    constexpr int RPS = 64 / C::KC;   // rows per store
#pragma unroll
    for (int t = 0; t < 32 / RPS; ++t) {
      const int row = RPS * t + lane / C::KC, ch = lane % C::KC;
      const int orow = __shfl(oi, row);   // lane `row` (hf = 0) holds that row's destination
      const uint4 val = *reinterpret_cast<const uint4 *>(obuf + row * (2 * D) + ((ch ^ (row % C::KC)) << 4));
      if (orow >= 0) *reinterpret_cast<uint4 *>(ob16 + (int64_t)orow * os2 + 8 * ch) = val;
    }
    if (lse_e && hf == 0 && oi >= 0) lse_e[bh * N + oi] = l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2 : -INFINITY;
  };
  if (kh == 0) half(std::integral_constant<int, 0>());
  else half(std::integral_constant<int, 1>());
}

}  // namespace pp
}  // namespace bsa
