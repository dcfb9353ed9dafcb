"""GPU parity of the query-head-pair path (bsa_attn_fwd with kv_share = 2):
grouped-query attention whose block pattern is shared by the query heads of a
KV group (INTRA, section 4: the Scatter/Gather prefill patterns hold for every
head), where one launch serves the identical rows of heads 2j and 2j + 1 and
stages each K/V tile once for both.

* bsa_schedule with head step 2 against the oracle's schedule, bit for bit.
* bsa_pair_rows_equal against the rows themselves (lists and log-weights).
* Attention on random group-identical masks (ragged N, causal, log-weights,
  query permutation with fused gather and scatter, lists longer than one LDS
  chunk, empty rows) against the oracle on sampled rows, at the tolerance of
  every attention test; the pipeline's "auto" choice is checked both ways.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api, pipeline
import synth
from parity_common import assert_within, compare_rows, oracle_csr, run_gpu, sample_rows

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def group_identical(w):
    """Copy the mask / threshold map / log-weight rows of head 2j onto head
    2j + 1 of every KV group."""
    nb = w.nQB
    for name in ("mask", "T", "lw_map"):
        a = getattr(w, name)
        if a is None:
            continue
        a = a.reshape(w.B, w.Hq // 2, 2, nb, -1)
        a[:, :, 1] = a[:, :, 0]
    return w


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", [
    (1, 4, 1, 37, 0, 8), (2, 8, 2, 50, 16, 8), (1, 32, 8, 64, 0, 8), (2, 4, 2, 300, 64, 3)])
def test_schedule_head_step_two_matches_oracle(B, Hq, Hkv, nQB, W, n_xcd):
    rng = np.random.default_rng(nQB)
    nnz = rng.integers(0, 40, size=B * Hq * nQB)
    rp = np.zeros(B * Hq * nQB + 1, dtype=np.int32)
    rp[1:] = np.cumsum(nnz)
    _log("case schedule head_step=2 B=%d Hq=%d Hkv=%d nQB=%d W=%d" % (B, Hq, Hkv, nQB, W))
    ref = oracle.schedule(rp, B, Hq, Hkv, nQB, W or 2048, n_xcd, head_step=2)
    got = api.schedule(torch.from_numpy(rp).cuda(), B, Hq, Hkv, nQB, W, n_xcd, head_step=2)
    np.testing.assert_array_equal(got.cpu().numpy(), ref)
    perm = np.stack([rng.permutation(nQB) for _ in range(B * Hq)]).astype(np.int32)
    ref = oracle.schedule(rp, B, Hq, Hkv, nQB, W or 2048, n_xcd, row_perm=perm, head_step=2)
    got = api.schedule(torch.from_numpy(rp).cuda(), B, Hq, Hkv, nQB, W, n_xcd, head_step=2,
                       row_perm=torch.from_numpy(perm).cuda())
    np.testing.assert_array_equal(got.cpu().numpy(), ref)


def test_pair_rows_equal():
    w = group_identical(synth.random_case(1200, B=2, Hq=4, Hkv=2, N=900, d=64, block=128, density=0.4,
                                          log_weights=True))
    rp, col, lw = oracle_csr(w)
    _log("case pair_rows_equal")
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    f = lambda c, l: int(api.pair_rows_equal(dev(rp), dev(c), w.B, w.Hq, w.Hkv, w.nQB, lw=l).item())
    assert f(col, dev(lw)) == 1
    assert f(col, None) == 1
    # a row of head 1 (b = 1, u = 3) with one block changed, then one log-weight
    r1 = (1 * w.Hq + 1) * w.nQB + 3
    assert rp[r1 + 1] > rp[r1]
    c2 = col.copy()
    c2[rp[r1]] = (c2[rp[r1]] + 1) % w.nQB
    assert f(c2, dev(lw)) == 0
    l2 = lw.copy()
    l2[rp[r1 + 1] - 1] += 1.0
    assert f(col, dev(l2)) == 0
    assert f(col, None) == 1
    # different lengths: the random masks of the workload before the copy
    w2 = synth.random_case(1201, B=1, Hq=4, Hkv=2, N=900, d=64, block=128, density=0.4)
    rp2, col2, _ = oracle_csr(w2)
    assert int(api.pair_rows_equal(dev(rp2), dev(col2), 1, 4, 2, w2.nQB).item()) == 0


CASES = {
    "d128_ragged": dict(B=1, Hq=4, Hkv=2, N=1000, d=128, block=128, density=0.4),
    "d64_gqa4": dict(B=2, Hq=4, Hkv=1, N=1200, d=64, block=128, density=0.5),
    "causal_gqa4": dict(B=1, Hq=8, Hkv=2, N=1500, d=128, block=128, density=0.6, causal=True),
    "log_weights": dict(B=1, Hq=4, Hkv=1, N=1100, d=128, block=128, density=0.5, log_weights=True),
    "permuted": dict(B=1, Hq=4, Hkv=2, N=1300, d=128, block=128, density=0.35, permute=True, n_clusters=6),
    "threshold_map": dict(B=1, Hq=4, Hkv=2, N=777, d=64, block=128, density=0.3, use_T=True),
    "single_partial": dict(B=1, Hq=2, Hkv=1, N=50, d=128, block=128, density=1.0, causal=True),
    "hot_queries": dict(B=1, Hq=4, Hkv=2, N=900, d=128, block=128, density=0.5, q_scale=8.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_kv_share_matches_oracle(name):
    w = group_identical(synth.random_case(1300 + list(CASES).index(name), **CASES[name]))
    _log("case kv_share %s" % name)
    _, res = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, kv_share="auto")
    assert res.kv_share
    assert res.order.numel() == w.B * w.Hq * w.nQB // 2
    pq = pk = None
    if w.permuted:
        pq = oracle.perm_from_labels(w.labels_q, w.n_clusters)
        pk = oracle.perm_from_labels(w.labels_k, w.n_clusters)
    rows = sample_rows(w, seed=7)
    stats = compare_rows(w, res, rows, pq, pk)
    _log("  %s" % stats)
    assert_within(stats)
    # without a launch table: launch i serves the i-th row of an even head
    _, r2 = run_gpu(w, schedule=False, kv_share=True)
    assert torch.equal(r2.out, res.out)
    assert torch.equal(r2.lse, res.lse)


def test_kv_share_empty_rows_and_long_lists():
    """Rows with no block (no forced diagonal) write O = 0 and LSE = -inf;
    rows of over a thousand blocks span several LDS list chunks."""
    w = synth.random_case(1400, B=1, Hq=2, Hkv=1, N=128 * 1100 - 45, d=128, block=128, density=0.97)
    w.force_diag = False
    w.mask = w.mask.reshape(1, 2, w.nQB, w.nQB)
    w.mask[0, :, 5] = 0
    w.mask[0, :, 700] = 0
    w = group_identical(w)
    w.mask = w.mask.reshape(-1, w.nQB)
    _log("case kv_share empty rows and long lists N=%d" % w.N)
    _, res = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, kv_share=True)
    assert np.diff(res.row_ptr.cpu().numpy()).max() > 1024
    rows = sample_rows(w, seed=8, per_block=False)
    rows = np.unique(np.concatenate([rows, np.arange(5 * 128, 6 * 128), w.N + np.arange(700 * 128, 701 * 128)]))
    stats = compare_rows(w, res, rows)
    _log("  %s" % stats)
    assert_within(stats)
    out = res.out.view(torch.int16).cpu().numpy().reshape(2, w.N, -1)
    assert np.all(out[:, 5 * 128:6 * 128] == 0)
    assert np.all(np.isneginf(res.lse.cpu().numpy().reshape(2, w.N)[:, 700 * 128:701 * 128]))


def test_auto_declines_rows_that_differ():
    w = synth.random_case(1500, B=1, Hq=4, Hkv=2, N=1000, d=128, block=128, density=0.4)
    _log("case kv_share auto on differing rows")
    _, res = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, kv_share="auto")
    assert not res.kv_share
    _, ref = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, kv_share=False)
    assert torch.equal(res.out, ref.out)


def test_prefill_pattern_gqa():
    """The LLM prefill pattern (local window of 4 blocks, stride-16 blocks, the
    first block; causal) at 32 query heads over 8 KV heads, 4096 tokens."""
    w = synth.llm_prefill(seed=6, Hq=32, Hkv=8, N=4096 - 77)
    _log("case kv_share prefill N=%d" % w.N)
    _, res = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0)
    assert res.kv_share
    rows = sample_rows(w, seed=9)
    stats = compare_rows(w, res, rows)
    _log("  %s" % stats)
    assert_within(stats)
