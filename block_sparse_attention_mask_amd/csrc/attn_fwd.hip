// bsa_attn_fwd: argument checks and dispatch to the attention kernels
// (dim-major V: attn_pp.hip for 128-key blocks, attn_dimv.hip for 64, and
// attn_ppg.hip for pairs of query heads that share K/V and their lists;
// token-major V: attn_tokv.hip; launch entries of rows and identical row
// pairs: attn_ppx in attn_ppg.hip).  Lists come as CSR or as CRM rows; the
// dim-major kernels have a variant for each.
#include "attn_common.h"

namespace {

bool bad_strides(const int64_t s[3]) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || (s[i] & 7)) return true;
  return false;
}

}  // namespace

extern "C" int bsa_attn_fwd(const bsa_attn_args *a, bsa_stream_t stream) {
  if (!a) return BSA_ERR_ARG;
  if (!a->q || !a->k || !a->v || !a->o) return BSA_ERR_ARG;
  if (!a->crm && (!a->row_ptr || !a->col)) return BSA_ERR_ARG;
  if (a->B <= 0 || a->Hq <= 0 || a->Hkv <= 0 || a->N <= 0 || a->n_order < 0) return BSA_ERR_ARG;
  if (a->Hq % a->Hkv) return BSA_ERR_ARG;
  if (a->v_layout != BSA_V_TOKEN_MAJOR && a->v_layout != BSA_V_DIM_MAJOR) return BSA_ERR_ARG;
  if ((a->d != 64 && a->d != 128) || (a->block != 64 && a->block != 128)) return BSA_ERR_UNSUPPORTED;
  if (a->causal && (a->scatter_perm_q || a->gather_perm_q)) return BSA_ERR_UNSUPPORTED;
  // CRM rows feed the dim-major kernels and carry no log-weights
  if (a->crm && (a->lw || a->v_layout != BSA_V_DIM_MAJOR)) return BSA_ERR_UNSUPPORTED;
  if (!bsa_aligned16(a->q) || !bsa_aligned16(a->k) || !bsa_aligned16(a->v) || !bsa_aligned16(a->o))
    return BSA_ERR_ARG;
  if (bad_strides(a->q_str) || bad_strides(a->k_str) || bad_strides(a->v_str) || bad_strides(a->o_str))
    return BSA_ERR_ARG;
  if (a->q_str[2] < a->d || a->k_str[2] < a->d || a->o_str[2] < a->d) return BSA_ERR_ARG;
  if (a->o == a->q || a->o == a->k || a->o == a->v) return BSA_ERR_ARG;
  const int64_t nQB = (a->N + a->block - 1) / a->block;
  const int64_t R = (int64_t)a->B * a->Hq * nQB;
  if (R >= (int64_t(1) << 31)) return BSA_ERR_UNSUPPORTED;
  const int64_t lim = int64_t(1) << 30;
  if (a->v_layout == BSA_V_DIM_MAJOR) {
    // rows of V^T must hold every key of the last block; per-head byte ranges
    // are addressed with buffer offsets below 2^30
    if (a->v_str[2] < nQB * a->block) return BSA_ERR_ARG;
    if (((a->N - 1) * a->q_str[2] + a->d) * 2 >= lim || ((a->N - 1) * a->k_str[2] + a->d) * 2 >= lim ||
        (int64_t)a->d * a->v_str[2] * 2 >= lim)
      return BSA_ERR_UNSUPPORTED;
  } else if (a->v_str[2] < a->d) {
    return BSA_ERR_ARG;
  }
  if (a->kv_share != 0 && a->kv_share != 2) return BSA_ERR_ARG;
  // launch entries that serve a row or an identical pair of rows
  if (a->order2 && !a->order) return BSA_ERR_ARG;
  if (a->order2 && (a->kv_share || a->crm || a->v_layout != BSA_V_DIM_MAJOR || a->block != 128))
    return BSA_ERR_UNSUPPORTED;
  const int G = a->Hq / a->Hkv;
  if (a->kv_share == 2 && (G % 2 || a->crm || a->v_layout != BSA_V_DIM_MAJOR || a->block != 128))
    return BSA_ERR_UNSUPPORTED;
  // with kv_share every launch serves a pair of rows
  const int64_t rows = a->kv_share == 2 ? R / 2 : R;
  const int64_t grid = a->order ? (a->n_order ? a->n_order : rows) : rows;
  if (grid > rows) return BSA_ERR_ARG;
  if (grid == 0) return BSA_OK;

  bsa::AttnParams p;
  p.q = static_cast<const uint16_t *>(a->q);
  p.k = static_cast<const uint16_t *>(a->k);
  p.v = static_cast<const uint16_t *>(a->v);
  p.o = static_cast<uint16_t *>(a->o);
  p.lse = a->lse;
  p.qs0 = a->q_str[0]; p.qs1 = a->q_str[1]; p.qs2 = a->q_str[2];
  p.ks0 = a->k_str[0]; p.ks1 = a->k_str[1]; p.ks2 = a->k_str[2];
  p.vs0 = a->v_str[0]; p.vs1 = a->v_str[1]; p.vs2 = a->v_str[2];
  p.os0 = a->o_str[0]; p.os1 = a->o_str[1]; p.os2 = a->o_str[2];
  p.row_ptr = a->row_ptr;
  p.col = a->col;
  p.crm = a->crm;
  p.crm_words = bsa_crm_words((int)nQB);
  p.crm_tail = bsa_crm_tail((int)nQB);
  p.lw = a->lw;
  p.order = a->order;
  p.order2 = a->order2;
  p.sperm = a->scatter_perm_q;
  p.gperm = a->gather_perm_q;
  p.N = a->N;
  p.R = R;
  p.Hq = a->Hq;
  p.G = G;
  p.nQB = (int)nQB;
  p.causal = a->causal ? 1 : 0;
  const float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->d);
  p.c = scale * bsa::kLog2e;

  hipStream_t s = bsa_hip_stream(stream);
  hipError_t err;
  if (a->v_layout == BSA_V_TOKEN_MAJOR) err = bsa::launch_attn_tokv(p, a->block, a->d, grid, s);
  else if (a->kv_share == 2) err = bsa::launch_attn_ppg(p, a->d, grid, s);
  else if (a->order2) err = bsa::launch_attn_ppx(p, a->d, grid, s);
  else if (a->block == 128) err = bsa::launch_attn_pp(p, a->d, grid, s);
  else err = bsa::launch_attn_dimv(p, a->block, a->d, grid, s);
  return err == hipSuccess ? BSA_OK : BSA_ERR_HIP;
}
