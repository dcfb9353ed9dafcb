"""GPU parity of the CRM path (ScalingAttention, section 7.2: Compressed Row
Mask rows; section 7.3: the forward iterator), called through the C ABI.

* bsa_crm_build words, bsa_crm_row_ptr offsets and bsa_crm_to_csr lists are
  compared bit for bit with the oracle's build_crm and crm_walk.
* Attention with CRM rows against the oracle on sampled rows (same tolerance
  as every attention test), and bit for bit against the CSR path on the same
  mask: both stage the same ascending list, so the kernels do the same
  arithmetic in the same order.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api
import synth
from parity_common import assert_within, compare_rows, run_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _mask_case(seed, R, nKB, density, use_T):
    rng = np.random.default_rng(seed)
    if use_T:
        T = rng.random((R, nKB), dtype=np.float32)
        T[1] = np.nan                      # never kept
        T[2] = -1.0                        # always kept
        return None, T, float(density)
    mask = (rng.random((R, nKB)) < density).astype(np.uint8)
    mask[1] = 0
    mask[2] = 7                            # any nonzero byte keeps
    return mask, None, 0.0


@pytest.mark.parametrize("nKB,density,use_T,force_diag", [
    (1, 0.5, False, True), (31, 0.3, False, False), (32, 0.5, True, True), (33, 0.2, False, True),
    (64, 0.9, True, False), (65, 0.05, False, False), (591, 0.2, False, True), (1100, 0.5, True, True)])
def test_crm_build_and_walk_bit_exact(nKB, density, use_T, force_diag):
    R = 3 * nKB + 5 if nKB < 100 else 2 * nKB
    mask, T, p = _mask_case(nKB, R, nKB, density, use_T)
    _log("case crm build nKB=%d R=%d use_T=%d force_diag=%d" % (nKB, R, use_T, force_diag))
    dmask = None if mask is None else torch.from_numpy(mask).cuda()
    dT = None if T is None else torch.from_numpy(T).cuda()
    g = api.crm_build(dmask, dT, p, nKB, force_diag)
    ref = oracle.build_crm(mask, T, p, nKB, force_diag)
    np.testing.assert_array_equal(g.cpu().numpy().view(np.uint32), ref)
    ref_rp, ref_col = oracle.crm_walk(ref, nKB)
    rp, nnz = api.crm_row_ptr(g, nKB)
    np.testing.assert_array_equal(rp.cpu().numpy(), ref_rp)
    assert nnz == ref_rp[-1]
    col = api.crm_to_csr(g, nKB, rp, nnz)
    np.testing.assert_array_equal(col.cpu().numpy(), ref_col)
    # the lists are the CSR builder's too
    csr_rp, csr_col, _ = oracle.build_csr(mask, T, p, None, nKB, force_diag)
    np.testing.assert_array_equal(ref_rp, csr_rp)
    np.testing.assert_array_equal(ref_col, csr_col)


def test_crm_padding_bits_ignored_and_capacity_respected():
    nKB, R = 40, 50                                      # last word holds blocks 32..39
    mask, _, _ = _mask_case(3, R, nKB, 0.4, False)
    ref = oracle.build_crm(mask, None, 0.0, nKB, False)
    junk = ref.copy()
    junk[:, 1] |= np.uint32(0xFFFFFF00)                  # bits for blocks 40..63
    _log("case crm padding bits and capacity")
    g = torch.from_numpy(junk.view(np.int32)).cuda()
    ref_rp, ref_col = oracle.crm_walk(ref, nKB)
    rp, nnz = api.crm_row_ptr(g, nKB)
    np.testing.assert_array_equal(rp.cpu().numpy(), ref_rp)
    cap = nnz // 2
    buf = torch.full((nnz + 8,), -5, dtype=torch.int32, device="cuda")
    check_rc = api.load().bsa_crm_to_csr(api._ptr(g), R, nKB, api._ptr(rp), api._ptr(buf), cap, None)
    assert check_rc == 0
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    np.testing.assert_array_equal(got[:cap], ref_col[:cap])
    assert np.all(got[cap:] == -5)


CRM_CASES = {
    "b64_d64_gqa_T": dict(B=2, Hq=4, Hkv=2, N=700, d=64, block=64, density=0.3, use_T=True),
    "b128_d128_causal_gqa": dict(B=1, Hq=4, Hkv=1, N=900, d=128, block=128, density=0.6, causal=True),
    "b128_d128_perm": dict(B=1, Hq=3, Hkv=3, N=1200, d=128, block=128, density=0.3, permute=True, n_clusters=7),
    "b64_d128_perm_gqa": dict(B=1, Hq=2, Hkv=1, N=777, d=128, block=64, density=0.35, permute=True),
    "b128_d64_full": dict(B=1, Hq=2, Hkv=2, N=640, d=64, block=128, density=2.0),
    "b128_d64_sparse_T": dict(B=1, Hq=2, Hkv=1, N=128 * 70 - 3, d=64, block=128, density=0.1, use_T=True),
    "single_partial_block": dict(B=1, Hq=2, Hkv=1, N=50, d=128, block=64, density=1.0, causal=True),
}


@pytest.mark.parametrize("name", list(CRM_CASES))
def test_crm_attention_matches_oracle_and_csr(name):
    w = synth.random_case(800 + list(CRM_CASES).index(name), **CRM_CASES[name])
    _log("case crm attention %s" % name)
    _, r_csr = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, pair_rows=False)
    _, r_crm = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, crm=True)
    assert torch.equal(r_crm.row_ptr, r_csr.row_ptr)
    # the CSR launch table may take the sequence order (the schedule sees the
    # lists); the CRM one sorts whole segments.  Outputs do not depend on it.
    rp_np = r_csr.row_ptr.cpu().numpy()
    assert np.array_equal(r_crm.order.cpu().numpy(), oracle.schedule(rp_np, w.B, w.Hq, w.Hkv, w.nQB, 0, 8))
    assert torch.equal(r_crm.out, r_csr.out)
    assert torch.equal(r_crm.lse, r_csr.lse)
    pq = pk = None
    if w.permuted:
        pq = oracle.perm_from_labels(w.labels_q, w.n_clusters)
        pk = oracle.perm_from_labels(w.labels_k, w.n_clusters)
    rows = sample_rows(w, seed=5)
    stats = compare_rows(w, r_crm, rows, pq, pk)
    _log("  %s" % stats)
    assert_within(stats)


@pytest.mark.parametrize("block,d,nblocks", [(128, 128, 1100), (64, 64, 1100)])
def test_crm_long_rows_span_list_chunks(block, d, nblocks):
    """Rows of over a thousand KV blocks: the CRM walk fills the LDS list one
    1024-entry chunk at a time, from a position inside a word batch."""
    w = synth.random_case(900 + block, B=1, Hq=2, Hkv=1, N=block * nblocks - 37, d=d, block=block, density=0.97)
    _log("case crm long rows block=%d d=%d N=%d" % (block, d, w.N))
    _, r_csr = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, pair_rows=False)
    _, r_crm = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, crm=True)
    assert np.diff(r_crm.row_ptr.cpu().numpy()).max() > 1024
    assert torch.equal(r_crm.out, r_csr.out)
    assert torch.equal(r_crm.lse, r_csr.lse)
    rows = sample_rows(w, seed=4, per_block=False)
    stats = compare_rows(w, r_crm, rows)
    _log("  %s" % stats)
    assert_within(stats)


def test_crm_stage1_schedule_matches_csr():
    w = synth.random_case(950, B=1, Hq=2, Hkv=2, N=1500, d=128, block=128, density=0.3)
    _log("case crm stage-1 schedule")
    _, r_csr = run_gpu(w, schedule=True, n_xcd=8, wave_rows=4, stage1="on", stage1_iters=6, pair_rows=False)
    _, r_crm = run_gpu(w, schedule=True, n_xcd=8, wave_rows=4, stage1="on", stage1_iters=6, crm=True)
    assert torch.equal(r_crm.order, r_csr.order)
    assert torch.equal(r_crm.out, r_csr.out)
