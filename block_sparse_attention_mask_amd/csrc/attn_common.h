// Internal: parameters and helpers shared by the attention kernels.
#pragma once
#include <type_traits>

#include "bsa_internal.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnParams {
  const uint16_t *q, *k, *v;
  uint16_t *o;
  float *lse;
  // element strides: q/k/o (batch, head, token); v (batch, head, token) when
  // token-major, (batch, head, head-dim row) when dim-major
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  const int32_t *row_ptr, *col;
  const uint32_t *crm;   // CRM rows in place of row_ptr/col (kernels instantiated for it)
  int crm_words;         // words per CRM row
  uint32_t crm_tail;     // bits of a row's last word that name KV blocks
  const float *lw;
  const int32_t *order;
  const int32_t *order2;  // second row of a launch entry (identical pair), or null
  const int32_t *sperm;
  const int32_t *gperm;  // query gather: permuted position -> row of q, or null
  int64_t N, R;
  int Hq, G, nQB, causal;
  float c;  // softmax scale * log2(e)
};

// The AttnParams of a kernel whose first argument it is, read through its
// kernel-argument block: the pointer passes through an empty asm statement,
// so each field is loaded where it is read (scalar loads) instead of being
// held in a scalar register from the kernel's start.
typedef const __attribute__((address_space(4))) AttnParams *kparams_t;
__device__ __forceinline__ kparams_t kernel_params() {
  kparams_t pk = (kparams_t)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(pk));
  return pk;
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOOR = 0x40000000u;     // offset past every buffer (extents < 2^30 bytes)
constexpr float kTau = 8.0f;               // lazy-rescale threshold (log2 units)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Key (within a 32-key M tile) held by MFMA row m of S^T.
__device__ __forceinline__ int key_of_row(int m) {
  return ((m >> 4) << 4) | (((m >> 2) & 1) << 3) | (((m >> 3) & 1) << 2) | (m & 3);
}

// Max and sum of a value over lanes l and l ^ 32 (the two halves of a
// wavefront hold different keys of the same queries).  The swap returns the
// upper half's value in the first result and the lower half's in the second,
// in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Chunk-position permutation of LDS row r (rows of `chunks` 16-byte chunks).
template <int chunks>
__device__ __forceinline__ int swz(int r) {
  static_assert(chunks == 8 || chunks == 16, "row width");
  return chunks == 16 ? (r & 15) : ((r >> 1) & 7);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (SGPR quad) for a byte range starting at base.
__device__ __forceinline__ i32x4 buffer_rsrc(const void *base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, kRsrcWord3};
}

// One 1 KB copy: 16 bytes per lane from buffer offset voff (+ soff) into LDS
// at lds + 16 lane.  Written as inline assembly so that the compiler does not
// track it (its waits are placed by hand at phase ends): M0 carries the LDS
// address; the nops cover the M0 and SGPR-operand hazards of a vector memory
// instruction.  No wavefront reads a buffer in the phase that refills it, and
// the phase barriers order everything else, so no memory clobber is needed.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voff),
               "s"(rsrc), "s"(soff)
               : "m0");
}

// The same copy with the LDS address formed in the instruction stream: M0 =
// base + IMM, so that a kernel keeps one SGPR of LDS base per wavefront
// instead of one per (buffer, copy slot).
template <uint32_t IMM>
__device__ __forceinline__ void lds_copy16_at(i32x4 rsrc, uint32_t base, uint32_t voff, uint32_t soff) {
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(base), "v"(voff),
               "s"(rsrc), "s"(soff), "n"(IMM)
               : "m0", "scc");
}
#pragma clang diagnostic pop

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt immediate (gfx9 encoding): at most n vector-memory operations of
// this wavefront outstanding, no LDS/scalar-memory operation outstanding,
// export counter not waited on.
constexpr int vm_lgkm0_wait_imm(int n) { return (n & 15) | (7 << 4) | (0 << 8) | ((n >> 4) << 14); }

hipError_t launch_attn_tokv(const AttnParams &p, int block, int d, int64_t grid, hipStream_t s);
hipError_t launch_attn_dimv(const AttnParams &p, int block, int d, int64_t grid, hipStream_t s);
hipError_t launch_attn_pp(const AttnParams &p, int d, int64_t grid, hipStream_t s);
hipError_t launch_attn_ppg(const AttnParams &p, int d, int64_t grid, hipStream_t s);
hipError_t launch_attn_ppx(const AttnParams &p, int d, int64_t grid, hipStream_t s);

}  // namespace bsa
