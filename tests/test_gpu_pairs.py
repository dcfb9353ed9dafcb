"""GPU tests of the paired launch tables (bsa_schedule_pairs) and of the
attention launch that serves a pair of identical rows in one entry
(bsa_attn_fwd with order2).

* The tables are bit-exact with oracle.schedule_pairs (shapes with GQA
  segments, buckets, the adaptive order, stage-1 row orders with a corrupt
  entry, log-weights).
* Attention through paired entries matches the oracle element by element on
  workloads whose consecutive query blocks repeat their lists (permuted with
  log-weights, causal, GQA, a partial last block, d = 64), and the clustered
  workload; it agrees with the one-row launch within rounding and repeats its
  own bits.
* Entries whose second row lies outside the rows serve the first row alone
  (the one-row body; equal to the one-row kernel's output within rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from block_sparse_attention_mask_amd import api
from parity_common import (assert_within, bf16_tensor_to_f32, compare_rows, oracle_csr, oracle_perms, run_gpu,
                           sample_rows)
from test_oracle_schedule_pairs import block_case

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


SCHED = [(1, 1, 1, 40, 0, 1), (2, 3, 3, 37, 0, 8), (1, 4, 2, 33, 0, 8), (1, 2, 2, 150, 64, 8),
         (2, 4, 1, 50, 16, 8), (1, 1, 1, 591, 0, 8), (1, 8, 8, 300, 0, 8)]


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", SCHED)
@pytest.mark.parametrize("with_lw", [False, True])
def test_schedule_pairs_bit_exact(B, Hq, Hkv, nQB, W, n_xcd, with_lw):
    rp, col, lw = block_case(nQB * 3 + Hq + (7 if with_lw else 0), B, Hq, Hkv, nQB, 4, with_lw)
    _log("case schedule pairs B=%d Hq=%d Hkv=%d nQB=%d W=%d xcd=%d lw=%s" % (B, Hq, Hkv, nQB, W, n_xcd, with_lw))
    d = lambda a: torch.from_numpy(a).cuda()
    o1, o2 = api.schedule_pairs(d(rp), d(col), B, Hq, Hkv, nQB, W, n_xcd, lw=None if lw is None else d(lw))
    r1, r2 = oracle.schedule_pairs(rp, col, B, Hq, Hkv, nQB, W, n_xcd, lw=lw)
    assert np.array_equal(o1.cpu().numpy(), r1)
    assert np.array_equal(o2.cpu().numpy(), r2)


def test_schedule_pairs_with_row_order_bit_exact():
    B, Hq, Hkv, nQB = 2, 4, 2, 60
    rp, col, _ = block_case(77, B, Hq, Hkv, nQB, 3)
    g = np.random.default_rng(5)
    perm = np.stack([g.permutation(nQB) for _ in range(B * Hq)]).astype(np.int32)
    perm[3, 7] = -1          # a corrupt stage-1 entry: its position serves nothing
    _log("case schedule pairs with a stage-1 order")
    d = lambda a: torch.from_numpy(a).cuda()
    for W in (0, 32):
        o1, o2 = api.schedule_pairs(d(rp), d(col), B, Hq, Hkv, nQB, W, 8, row_perm=d(perm))
        r1, r2 = oracle.schedule_pairs(rp, col, B, Hq, Hkv, nQB, W, 8, row_perm=perm)
        assert np.array_equal(o1.cpu().numpy(), r1)
        assert np.array_equal(o2.cpu().numpy(), r2)


def repeat_rows(w, seed, max_run=4):
    """Copy each head's mask (and log-weight) rows so that consecutive query
    blocks list the same blocks in runs of 1..max_run; the forced diagonal
    keeps the run's own blocks listed."""
    g = np.random.default_rng(seed)
    R, nb = w.mask.shape
    m = w.mask.copy()
    lwm = None if w.lw_map is None else w.lw_map.copy()
    for h0 in range(0, R, w.nQB):
        u = 0
        while u < w.nQB:
            n = int(g.integers(1, max_run + 1))
            rows = list(range(h0 + u, min(h0 + u + n, h0 + w.nQB)))
            src = m[rows[0]].copy()
            for r in rows:
                src[r - h0] = 1              # every diagonal of the run in every row of it
            for r in rows:
                m[r] = src
                if lwm is not None:
                    lwm[r] = lwm[rows[0]]
            u += n
    w.mask = m
    w.lw_map = lwm
    return w


CASES = {
    "perm_lw": dict(B=1, Hq=2, Hkv=2, N=2000, d=128, block=128, density=0.3, permute=True, log_weights=True),
    "causal_gqa": dict(B=1, Hq=4, Hkv=2, N=1700, d=128, block=128, density=0.4, causal=True),
    "tail_d64": dict(B=2, Hq=2, Hkv=1, N=1111, d=64, block=128, density=0.35),
    "perm_gqa_lw": dict(B=1, Hq=4, Hkv=1, N=1500, d=128, block=128, density=0.25, permute=True, log_weights=True,
                        n_clusters=7),
}


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("overlap", [False, True])
def test_paired_attention_matches_oracle(name, overlap):
    w = repeat_rows(synth.random_case(1500 + list(CASES).index(name), **CASES[name]), 3)
    _log("case paired attention %s overlap=%s" % (name, overlap))
    _, res = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, overlap=overlap)
    assert res.order2 is not None
    n_pairs = int((res.order2 >= 0).sum().item())
    R = w.B * w.Hq * w.nQB
    assert n_pairs > R // 5, n_pairs
    rp, col, lw = oracle_csr(w)
    o1, o2 = oracle.schedule_pairs(rp, col, w.B, w.Hq, w.Hkv, w.nQB, 0, 8, lw=lw)
    assert np.array_equal(res.order.cpu().numpy(), o1) and np.array_equal(res.order2.cpu().numpy(), o2)
    pq, pk = oracle_perms(w)
    rows = np.arange(w.B * w.Hq * w.N, dtype=np.int64)
    stats = compare_rows(w, res, rows, pq, pk)
    _log("  %d pairs of %d rows; %s" % (n_pairs, R, stats))
    assert_within(stats)
    # the one-row launch computes the same function (key halves merged at the
    # end instead of one softmax state over all keys): equal within rounding
    _, single = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, overlap=overlap, pair_rows=False)
    assert single.order2 is None
    diff = np.abs(bf16_tensor_to_f32(single.out) - bf16_tensor_to_f32(res.out))
    assert float(diff.max()) <= 2e-2
    # the same tables give the same bits
    _, again = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, overlap=overlap)
    assert torch.equal(again.out, res.out) and torch.equal(again.lse, res.lse)


def test_paired_attention_clustered_workload():
    """The clustered workload's lists at a reduced shape (4 heads x 16384
    tokens, 16 clusters): most rows pair up; sampled rows against the
    oracle."""
    w = synth.clustered(H=4, N=16384, C=16)
    _log("case paired attention, clustered 4 x 16384")
    _, res = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, overlap=True)
    n_pairs = int((res.order2 >= 0).sum().item())
    assert 2 * n_pairs > 0.8 * w.B * w.Hq * w.nQB
    pq, pk = oracle_perms(w)
    rows = sample_rows(w, seed=9)
    stats = compare_rows(w, res, rows, pq, pk)
    _log("  %d pairs; %s" % (n_pairs, stats))
    assert_within(stats)


def test_second_row_outside_the_rows_serves_the_first_alone():
    """Launch entries whose order2 lies outside [0, R) (negative or past the
    rows) serve row order[i] alone, with the one-row body: every row is
    written, equal to the one-row kernel's output within rounding."""
    w = synth.random_case(1600, B=1, Hq=3, Hkv=3, N=1300, d=128, block=128, density=0.4, log_weights=True)
    dw, single = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, pair_rows=False)
    R = w.B * w.Hq * w.nQB
    _log("case order2 outside the rows")
    v = api.transpose_rows(dw.v, None, ld=dw.nQB * dw.block)
    order2 = torch.where(torch.arange(R, device="cuda") % 2 == 0, torch.full((R,), -3, device="cuda"),
                         torch.full((R,), R + 5, device="cuda")).to(torch.int32)
    out, lse = api.attn_fwd(dw.q, dw.k, v, single.row_ptr, single.col, dw.block, lw=single.lw, order=single.order,
                            order2=order2, want_lse=True, v_dim_major=True)
    torch.cuda.synchronize()
    assert float(np.abs(bf16_tensor_to_f32(out) - bf16_tensor_to_f32(single.out)).max()) <= 2e-3
    assert float((lse - single.lse).abs().max()) <= 1e-4
