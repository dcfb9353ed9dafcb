// Internal: parameters and helpers shared by the attention kernels.
#pragma once
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
  const float *lw;
  const int32_t *order;
  const int32_t *sperm;
  int64_t N, R;
  int Hq, G, nQB, causal;
  float c;  // softmax scale * log2(e)
};

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

hipError_t launch_attn_tokv(const AttnParams &p, int block, int d, int64_t grid, hipStream_t s);
hipError_t launch_attn_dimv(const AttnParams &p, int block, int d, int64_t grid, hipStream_t s);

}  // namespace bsa
