// Block-sparse softmax attention forward for CDNA4 (gfx950), 128-query
// blocks, V dim-major: the plain kernels of the ping-pong body in
// attn_pp_body.h (one workgroup per CSR row), for each head dim and list
// format (CSR lists, or CRM words).
#include "attn_pp_body.h"

namespace bsa {
namespace pp {

// One plain kernel per head dim and list format.  The body reads some of its
// arguments again through the kernel's argument block, so the AttnParams is
// the first argument.  A launch-table entry outside the rows computes
// nothing.
#define BSA_PP_KERNEL(NAME, D, CRM)                                                                 \
  __global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))     \
  void NAME(const AttnParams p, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ col, \
            const float *__restrict__ lw, const int32_t *__restrict__ order,                         \
            const int32_t *__restrict__ sperm, uint16_t *__restrict__ out, float *__restrict__ lse) { \
    __shared__ PpShared<D> sh;                                                                      \
    const int32_t r = order ? order[blockIdx.x] : (int32_t)blockIdx.x;                             \
    if (r < 0 || r >= p.R) return;                                                                 \
    attn_pp_body<D, CRM>(p, sh, r, row_ptr, col, lw, sperm, out, lse);                              \
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
