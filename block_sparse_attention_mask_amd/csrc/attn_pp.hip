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
  static constexpr int NSK = NKC / NW, NSV = NVC / NW;
  static constexpr int NSLOT = NSK + NSV;           // copies per wavefront per phase
  static constexpr int KB = NKC * 1024, VB = NVC * 1024;
  static constexpr int NM = MTW * (2 * DT + KS);    // MFMAs per matrix step
  static constexpr int LIST = 1024;                 // CSR entries staged in LDS at a time
  static_assert(NKC % NW == 0 && NVC % NW == 0, "whole copies per wavefront");
  static_assert(NM % NSLOT == 0, "copies spread evenly over the matrix step");
  static_assert((2 * MTW) % NSLOT == 0 || NSLOT % (2 * MTW) == 0, "copies spread evenly over the softmax step");
  static_assert(64 * DT * 16 * 4 <= KB, "merge data of a query group fits a K buffer");
};

template <int D, bool kCrm>
__device__ __forceinline__ void attn_pp_body(const AttnParams &p, const int32_t *__restrict__ row_ptr,
                                             const int32_t *__restrict__ col, const float *__restrict__ lw,
                                             const int32_t *__restrict__ order,
                                             const int32_t *__restrict__ sperm, uint16_t *__restrict__ out,
                                             float *__restrict__ lse) {
  using C = PCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint8_t kx0[C::KB], kx1[C::KB], ky0[C::KB], ky1[C::KB];
  __shared__ __attribute__((aligned(1024))) uint8_t vx0[C::VB], vx1[C::VB], vy0[C::VB], vy1[C::VB];
  __shared__ int32_t lcol[C::LIST];
  __shared__ float lbias[C::LIST];
  __shared__ float mrg_ml[C::NQG][2][64];

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

  // Copy slots.  Slot t of wavefront w is copy c = w + 8 t of a phase: K copy
  // c for t < NSK, else V^T copy c - NKC.  Copy c writes LDS bytes
  // [1024 c, 1024 c + 1024) of its buffer; lane l writes LDS slot 64 c + l,
  // which holds (row, chunk position) = divmod(slot, row chunks), so the lane
  // reads source chunk position ^ swz(row).  lo[t] is that source offset
  // within the half tile.
  uint32_t lo[C::NSLOT];
#pragma unroll
  for (int t = 0; t < C::NSLOT; ++t) {
    const int c = wave + C::NW * t;
    if (t < C::NSK) {
      const int s = c * 64 + lane, row = s / C::KC, ch = (s % C::KC) ^ swz<C::KC>(row);
      lo[t] = (uint32_t)row * ks2b + ch * 16;
    } else {
      const int s = (c - C::NKC) * 64 + lane, row = s / C::VC, ch = (s % C::VC) ^ swz<C::VC>(row);
      lo[t] = (uint32_t)row * vs2b + ch * 16;
    }
  }
  auto lds_addr = [](const uint8_t *ptr) -> uint32_t {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)ptr;
  };

  int n = 0;   // entries of the current list chunk
  // Source offsets of a phase's half tiles: K entry ki and V^T entry vi of
  // half hh.  Entries outside [0, n) read zeros (offsets past the buffer).
  struct Src {
    uint32_t kbase, vso, vadd;
  };
  auto src_of = [&](int hh, int ki, int vi) -> Src {
    const bool kin = (uint32_t)ki < (uint32_t)n, vin = (uint32_t)vi < (uint32_t)n;
    const uint32_t kb = (uint32_t)lcol[kin ? ki : 0], vb = (uint32_t)lcol[vin ? vi : 0];
    const uint32_t kblk = __builtin_amdgcn_readfirstlane(kb < (uint32_t)p.nQB ? kb : 0u);
    const uint32_t vblk = __builtin_amdgcn_readfirstlane(vb < (uint32_t)p.nQB ? vb : 0u);
    Src sr;
    sr.kbase = kin ? (kblk * C::BLK + C::HK * hh) * ks2b : kOOR;
    sr.vso = vin ? (vblk * C::BLK + C::HK * hh) * 2 : 0u;
    sr.vadd = vin ? 0u : kOOR;
    return sr;
  };
  auto copy_slot = [&](int t, uint8_t *kdst, uint8_t *vdst, const Src &sr) {
    const int c = wave + C::NW * t;
    if (t < C::NSK) lds_copy16(krs, lds_addr(kdst) + c * 1024, lo[t] + sr.kbase, 0u);
    else lds_copy16(vrs, lds_addr(vdst) + (c - C::NKC) * 1024, lo[t] + sr.vadd, sr.vso);
  };

  // End of a phase: this wavefront's LDS reads are done and its copies from
  // two phases ago have landed; then the barrier.  The empty asm statements
  // keep the compiler from moving memory accesses across the barrier.
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto end_phase = [&]() {
    __builtin_amdgcn_s_waitcnt(vm_lgkm0_wait_imm(2 * C::NSLOT));
    barrier();
  };

  // Everything from here on is instantiated per key half (KH = kh), so that
  // each half's accumulators live in one set of registers and every LDS
  // buffer a step touches is a known object.
  auto half = [&](auto khc) {
    constexpr int KH = decltype(khc)::value;
    float m_run = 0.f, l_run = 0.f;
    f32x16 o[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    f32x16 s[C::MTW];
    bf16x8 pb[C::MTW][2];
#pragma unroll
    for (int jj = 0; jj < C::MTW; ++jj) pb[jj][0] = pb[jj][1] = bf16x8{};

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
      asm volatile("" ::"v"(m_run), "v"(l_run));
    };

    // Matrix step: O += V^T P^T (previous tile), then S = K Q^T (this tile);
    // one 16-byte LDS read per MFMA, the phase's copies spread between them.
    // Before the first tile pb is zero and the V^T buffer holds zeros; after
    // the last one S is not used.
    auto mstep = [&](const uint8_t *vt, const uint8_t *kt, uint8_t *kd, uint8_t *vd, const Src &sr) {
      constexpr int every = C::NM / C::NSLOT;
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) {
            const uint4 a = *reinterpret_cast<const uint4 *>(vt + ((va ^ (64 * jj + 32 * s2)) + 4096 * dt));
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb[jj][s2], o[dt], 0, 0, 0);
            const int m = (jj * 2 + s2) * C::DT + dt + 1;
            if (m % every == 0) copy_slot(m / every - 1, kd, vd, sr);
          }
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[jj][i] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj) {
          const uint4 a = *reinterpret_cast<const uint4 *>(kt + (ka[jj] ^ (32 * ks)));
          s[jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[jj], 0, 0, 0);
          const int m = 2 * C::MTW * C::DT + ks * C::MTW + jj + 1;
          if (m % every == 0) copy_slot(m / every - 1, kd, vd, sr);
        }
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

    // softmax step of list entry i: mask, max, lazy rescale, exponentials -> pb,
    // with the phase's copies spread over the four groups of eight
    // exponentials
    auto estep = [&](int i, uint8_t *kd, uint8_t *vd, const Src &sr) {
      const uint32_t vb = (uint32_t)lcol[i];
      const float bias = lbias[i];
      if (vb >= (uint32_t)mlim) {
        asm volatile("");   // keep this a branch: most tiles need no mask
        // keys past N (last block) and, when causal, keys after the query; a
        // block index outside the rows masks every key.  Element e of M tile
        // jj holds key offset ob + 32 jj + 16 (e >> 3) + (e & 7) in the block.
        const int vbc = vb < (uint32_t)p.nQB ? (int)vb : p.nQB;
        const int kbase = vbc * C::BLK;
        const int lim_n = N - kbase > C::BLK ? C::BLK : (N - kbase < 0 ? 0 : N - kbase);   // offsets >= lim_n: padding
        const int lc = p.causal ? qi - kbase + 1 : C::BLK;                                  // offsets >= lc: after the query
        const int lim = (lc < lim_n ? lc : lim_n) - ob;
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (32 * jj + 16 * (e >> 3) + (e & 7) >= lim) s[jj][e] = -INFINITY;
      }
      // exponentials against the running max; it is moved only when a lane's
      // 32 probabilities sum past 32 * 2^8 (some probability above 2^8) or
      // the lane's sum so far is below 2^-64, and then the tile is redone
      float nb = bias - m_run;
      float ls = 0.f;
#pragma unroll
      for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          float pv[8];
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8) pv[e8] = __builtin_amdgcn_exp2f(fmaf(s[jj][8 * s2 + e8], p.c, nb));
          ls += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
          pb[jj][s2] = __builtin_bit_cast(bf16x8, make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                                                             cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7])));
          const int gi = 2 * jj + s2;   // exponential group; its copies follow it
          asm volatile("" ::"v"(pb[jj][s2]));
#pragma unroll
          for (int t = gi * C::NSLOT / (2 * C::MTW); t < (gi + 1) * C::NSLOT / (2 * C::MTW); ++t)
            copy_slot(t, kd, vd, sr);
        }
      if (__any(ls > 32.f * 256.f || l_run + ls < 0x1p-64f)) {
        float m = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
          for (int e = 0; e < 16; ++e) m = fmaxf(m, fmaf(s[jj][e], p.c, nb));
        m = halves_max(m);
        const float lsum = halves_sum(ls), lrun = halves_sum(l_run);
        // Raised when a probability may exceed 2^8.  While the sum so far
        // (this tile included) is below 2^-64 (nothing, or only denormal
        // probabilities), moved toward the tile max: all the way when nothing
        // has been accumulated (O and l are zero and are multiplied by 0), by
        // at most 64 otherwise, so the rescale factor stays finite.
        float sh = 0.f;
        if (m > kTau) sh = m;
        else if (lrun + lsum < 0x1p-64f && m > -INFINITY) sh = lrun == 0.f ? m : fmaxf(m, -64.f);
        m_run += sh;
        nb = bias - m_run;
        const float alpha = lrun == 0.f ? 0.f : __builtin_amdgcn_exp2f(-sh);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
        ls = 0.f;
#pragma unroll
        for (int jj = 0; jj < C::MTW; ++jj)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            float pv[8];
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) pv[e8] = __builtin_amdgcn_exp2f(fmaf(s[jj][8 * s2 + e8], p.c, nb));
            ls += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
            pb[jj][s2] = __builtin_bit_cast(bf16x8, make_uint4(cvt_pk_bf16(pv[0], pv[1]), cvt_pk_bf16(pv[2], pv[3]),
                                                               cvt_pk_bf16(pv[4], pv[5]), cvt_pk_bf16(pv[6], pv[7])));
          }
      }
      l_run += ls;
    };

    // Phase loop.  Half 0 runs M(0) E(0) M(1) ... E(n-1) M(n) in phases
    // 0 .. 2n and idles in phase 2n+1; half 1 idles in phase 0 and runs the
    // same steps in phases 1 .. 2n+1.  M(j) reads V^T entry j-1 of this half
    // from vmine[(j-1) & 1] and K entry j from kmine[j & 1].  Copies of phase
    // f: half (f odd ? 0 : 1), K entry (f+3)/2 into that half's K buffer
    // (entry & 1), V^T entry (f+1)/2 into its V^T buffer (entry & 1).  In
    // phase 2n+1 only half 1 copies (entries past the list, never read).
    uint8_t *const km0 = KH ? ky0 : kx0, *const km1 = KH ? ky1 : kx1;
    uint8_t *const vm0 = KH ? vy0 : vx0, *const vm1 = KH ? vy1 : vx1;
    auto m_phase = [&](int j, auto par) {
      constexpr int P = decltype(par)::value;   // j & 1
      // phase 2j + KH: half 0 copies into half 1's buffers and vice versa
      uint8_t *kd, *vd;
      int hh, ki, vi;
      if (KH == 0) {   // phase 2j: half 1, K entry j+1, V^T entry j
        kd = P ? ky0 : ky1;
        vd = P ? vy1 : vy0;
        hh = 1, ki = j + 1, vi = j;
      } else {         // phase 2j+1: half 0, K entry j+2, V^T entry j+1
        kd = P ? kx1 : kx0;
        vd = P ? vx0 : vx1;
        hh = 0, ki = j + 2, vi = j + 1;
      }
      const Src sr = src_of(hh, ki, vi);
      mstep(P ? vm0 : vm1, P ? km1 : km0, kd, vd, sr);
      pin_results();
      end_phase();
    };
    auto e_phase = [&](int j, auto par) {
      constexpr int P = decltype(par)::value;
      // phase 2j+1+KH: this half, K entry j+2 into kmine[j & 1], V^T entry
      // j+1 into vmine[(j+1) & 1]
      const Src sr = src_of(KH, j + 2, j + 1);
      estep(j, P ? km1 : km0, P ? vm0 : vm1, sr);
      pin_results();
      end_phase();
    };
    auto run_half = [&]() {
      using Z = std::integral_constant<int, 0>;
      using O = std::integral_constant<int, 1>;
      if (KH == 1) {   // phase 0: half 1, K entry 1 into ky1, V^T entry 0 into vy0
        const Src sr = src_of(1, 1, 0);
#pragma unroll
        for (int t = 0; t < C::NSLOT; ++t) copy_slot(t, ky1, vy0, sr);
        end_phase();
      }
      for (int j = 0;; j += 2) {
        m_phase(j, Z());
        if (j == n) break;
        e_phase(j, Z());
        m_phase(j + 1, O());
        if (j + 1 == n) break;
        e_phase(j + 1, O());
      }
      if (KH == 0) barrier();   // phase 2n+1
    };

    for (int c0 = e0; c0 < e1; c0 += C::LIST) {
      n = e1 - c0 < C::LIST ? e1 - c0 : C::LIST;
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
      // what the first phases read: K entries 0 and 1 and V^T entry 0 of half
      // 0, K entry 0 of half 1, and zeros for "V^T entry -1" of both halves
      // (all eight wavefronts copy, as in a phase)
      {
        const Src s0 = src_of(0, 0, 0), s1 = src_of(0, 1, -1), s2 = src_of(1, 0, -1);
#pragma unroll
        for (int t = 0; t < C::NSLOT; ++t) {
          copy_slot(t, kx0, vx0, s0);
          copy_slot(t, kx1, vx1, s1);
          copy_slot(t, ky0, vy1, s2);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      run_half();
      __builtin_amdgcn_s_waitcnt(0);   // every copy has landed before the buffers are reused
      __syncthreads();
    }

    // merge the two key halves of every query group, normalise, store
    const float l_w = halves_sum(l_run);
    uint8_t *const mbuf = qg == 0 ? kx0 : qg == 1 ? kx1 : qg == 2 ? ky0 : ky1;
    float *scratch = reinterpret_cast<float *>(mbuf);
    if (KH == 1) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<f32x4 *>(scratch + ((dt * 4 + i4) * 64 + lane) * 4) =
              f32x4{o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]};
      mrg_ml[qg][0][lane] = m_run;
      mrg_ml[qg][1][lane] = l_w;
    }
    __syncthreads();
    if (KH != 0) return;
    const float m2 = mrg_ml[qg][0][lane];
    const float l2 = mrg_ml[qg][1][lane];
    // A half with nothing accumulated (l = 0) takes no part, whatever running
    // max it holds: its max may sit far above the other half's (a fully
    // masked half keeps its starting max of 0 while the other half's scores
    // are far below it), and a weight 2^(m_other - m) would then underflow.
    const float m = l_w > 0.f ? (l2 > 0.f ? fmaxf(m_run, m2) : m_run) : m2;
    const float a1 = l_w > 0.f ? __builtin_amdgcn_exp2f(m_run - m) : 0.f;
    const float a2 = l2 > 0.f ? __builtin_amdgcn_exp2f(m2 - m) : 0.f;
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
  };
  if (kh == 0) half(std::integral_constant<int, 0>());
  else half(std::integral_constant<int, 1>());
}

// One plain kernel per head dim and list format (CSR, or CRM words).
#define BSA_PP_KERNEL(NAME, D, CRM)                                                                 \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))     \
  void NAME(const AttnParams p, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col, \
            const float *__restrict__ lw, const int32_t *__restrict__ order,                         \
            const int32_t *__restrict__ sperm, uint16_t *__restrict__ out, float *__restrict__ lse) { \
    attn_pp_body<D, CRM>(p, row_ptr, col, lw, order, sperm, out, lse);                             \
  }
BSA_PP_KERNEL(attn_pp_128_128, 128, false)
BSA_PP_KERNEL(attn_pp_128_64, 64, false)
BSA_PP_KERNEL(attn_pp_crm_128_128, 128, true)
BSA_PP_KERNEL(attn_pp_crm_128_64, 64, true)
#undef BSA_PP_KERNEL

}  // namespace pp

hipError_t launch_attn_pp(const AttnParams &p, int d, int64_t grid, hipStream_t s) {
  const dim3 g((unsigned)grid), t(512);
#define BSA_ARGS p, p.row_ptr, p.col, p.lw, p.order, p.sperm, p.o, p.lse
  if (p.crm) {
    if (d == 128) hipLaunchKernelGGL(pp::attn_pp_crm_128_128, g, t, 0, s, BSA_ARGS);
    else hipLaunchKernelGGL(pp::attn_pp_crm_128_64, g, t, 0, s, BSA_ARGS);
  } else if (d == 128) {
    hipLaunchKernelGGL(pp::attn_pp_128_128, g, t, 0, s, BSA_ARGS);
  } else {
    hipLaunchKernelGGL(pp::attn_pp_128_64, g, t, 0, s, BSA_ARGS);
  }
#undef BSA_ARGS
  return hipGetLastError();
}

}  // namespace bsa
