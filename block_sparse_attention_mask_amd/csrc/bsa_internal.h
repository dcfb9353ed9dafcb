// Internal helpers shared by the library's HIP translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsattn.h"

#define BSA_LAUNCH_CHECK()                        \
  do {                                            \
    if (hipGetLastError() != hipSuccess) return BSA_ERR_HIP; \
  } while (0)

#define BSA_HIP(call)                             \
  do {                                            \
    if ((call) != hipSuccess) return BSA_ERR_HIP; \
  } while (0)

static inline hipStream_t bsa_hip_stream(bsa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

static inline bool bsa_aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Wave-wide helpers (wavefront size 64 on CDNA).
__device__ __forceinline__ uint64_t bsa_lanemask_lt(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int bsa_wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ int bsa_wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// CRM rows (ScalingAttention, section 7.2): ceil(nKB / 32) uint32 words per
// row, bit v % 32 of word v / 32 set when KV block v is listed.  Bits of the
// last word at v >= nKB are not part of the row.
__host__ __device__ __forceinline__ int bsa_crm_words(int nKB) { return (nKB + 31) / 32; }
__host__ __device__ __forceinline__ uint32_t bsa_crm_tail(int nKB) {
  return (nKB & 31) ? (1u << (nKB & 31)) - 1u : ~0u;
}

// Word w of a CRM row with the padding bits cleared (0 past the row).
__device__ __forceinline__ uint32_t bsa_crm_word(const uint32_t *row, int w, int W, uint32_t tail) {
  if (w >= W) return 0u;
  const uint32_t x = row[w];
  return w == W - 1 ? x & tail : x;
}

// Number of blocks in a CRM row (every lane of the wavefront gets it).
__device__ __forceinline__ int bsa_crm_count(const uint32_t *row, int W, uint32_t tail, int lane) {
  int c = 0;
  for (int w = lane; w < W; w += 64) c += __popc(bsa_crm_word(row, w, W, tail));
  return bsa_wave_sum(c);
}

// Ascending walk of a CRM row (ScalingAttention, section 7.3, forward
// iterator): positions [c0, c0 + lim) of the row's block list go to
// dst[position - c0].  The words are taken 64 at a time, one per lane; a
// scan of their popcounts gives each word's first list position, and the
// wavefront walks the bits of its word that `part`/`nparts` selects (a
// contiguous 32/nparts-bit slice, so nparts wavefronts together cover the
// word) by count-trailing-zeros and clear-lowest-bit.  Every wavefront of a
// group must call it with the same arguments except `part`.  Returns the
// number of blocks it passed over: the row's length whenever that is below
// c0 + lim (the walk stops at the first word batch that reaches c0 + lim).
__device__ __forceinline__ int bsa_crm_walk(const uint32_t *row, int W, uint32_t tail, int c0, int lim,
                                            int32_t *dst, int part, int nparts, int lane) {
  const int sb = 32 / nparts;
  const uint32_t below = (1u << (sb * part)) - 1u;
  const uint32_t mine = (sb == 32 ? ~0u : (1u << sb) - 1u) << (sb * part);
  int run = 0;   // list position of the batch's first block
  for (int w0 = 0; w0 < W && run < c0 + lim; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t x = bsa_crm_word(row, w, W, tail);
    const int cnt = __popc(x);
    const int incl = bsa_wave_incl_scan(cnt, lane);
    int pos = run + (incl - cnt) + __popc(x & below);
    for (uint32_t y = x & mine; y; y &= y - 1u, ++pos) {
      const int i = pos - c0;
      if (i >= 0 && i < lim) dst[i] = 32 * w + __builtin_ctz(y);
    }
    run += __shfl(incl, 63, 64);
  }
  return run;
}
