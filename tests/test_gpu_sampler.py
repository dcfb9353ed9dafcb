"""GPU parity of the group-shared importance sampler (InstaGen, Algorithm 1
steps 2-13 at tile granularity) and of the centroids it scores, called
through the C ABI.

* segment offsets: bit for bit against the oracle.
* segment means: fp32 sums on the device against the oracle's fp64 means
  (rtol 1e-5, atol 2e-6).
* sampler: on the same inputs, the mask must match the oracle's bit for bit
  and the log-weights within 1e-6.  Both sides decide in fp64, summing in
  different orders; a decision may differ only where the oracle's own margin
  is below 1e-9 (an exact-set boundary between two masses that equal to
  1e-9, or a systematic-PPS point within 1e-9 of a running-sum boundary),
  and the test checks that margin for every group that differs.
* the sampled pipeline end to end (device centroids, sampler, CSR, attention)
  against the oracle chain on small permuted workloads.
"""
import time

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api, pipeline
import synth
from parity_common import assert_within, compare_rows, sample_rows

pytestmark = pytest.mark.gpu

TIE = 1e-9


def _log(msg):
    print(msg, flush=True)


def _gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _problem(seed, B, Hq, Hkv, N, block, d, G, spread):
    rng = np.random.default_rng(seed)
    nb = -(-N // block)
    qbar = (rng.standard_normal((B * Hq, G, d)) * spread).astype(np.float32)
    kbar = (rng.standard_normal((B * Hkv, nb, d)) * spread).astype(np.float32)
    labels = rng.integers(0, G, size=(B * Hq, N)).astype(np.int32)
    seg = oracle.segment_offsets(labels, G)
    uoff = rng.random((B * Hq, G))
    return qbar, kbar, seg, uoff


def _margin(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, m_sample, pi, bh, g):
    """The oracle's smallest decision margin for group (bh, g)."""
    d = qbar.shape[2]
    nb = kbar.shape[1]
    b, h = divmod(bh, Hq)
    a = kbar[b * Hkv + h // (Hq // Hkv)].astype(np.float64) @ qbar[bh, g].astype(np.float64) / np.sqrt(d)
    mass = np.minimum(block, N - np.arange(nb) * block) * np.exp(a - a.max())
    srt = np.sort(mass)[::-1]
    ne = min(m_exact, nb)
    gaps = [1.0]
    if 0 < ne < nb:
        gaps.append(abs(srt[ne - 1] - srt[ne]) / srt[ne - 1])
    order = np.lexsort((np.arange(nb), -mass))
    resid = np.sort(order[ne:])
    c = np.cumsum(pi[bh, g, resid])
    pts = uoff[bh, g] + np.arange(m_sample)
    if len(c):
        gaps.append(np.abs(c[:, None] - pts[None, :]).min())
    return min(gaps)


def _compare_sampler(args, got, ref, label):
    qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, m_sample = args
    gm, glw, gpi = got
    om, olw, opi = ref
    nb = kbar.shape[1]
    G = qbar.shape[1]
    # groups whose decisions differ: by their rows' masks or by their pi
    groups = set()
    for r in np.nonzero((gm != om).any(1))[0]:
        bh, u = divmod(int(r), nb)
        groups.add((bh, int(np.searchsorted(seg[bh], u * block, side="right") - 1)))
    pi_bad = ~np.isclose(gpi, opi, rtol=1e-12, atol=1e-15).all(2)
    for bh, g in zip(*np.nonzero(pi_bad)):
        groups.add((int(bh), int(g)))
    for bh, g in groups:
        m = _margin(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, m_sample, opi, bh, g)
        assert m < TIE, "group (%d, %d) differs with decision margin %.3g" % (bh, g, m)
    same = np.ones(gm.shape[0], bool)
    for bh, g in groups:
        u0 = -(-int(seg[bh, g]) // block)
        u1 = min(nb, -(-int(seg[bh, g + 1]) // block))
        same[bh * nb + u0:bh * nb + u1] = False
    np.testing.assert_array_equal(gm[same], om[same])
    np.testing.assert_allclose(glw[same], olw[same], rtol=0, atol=1e-6)
    assert G > 0
    _log("  %s: %d rows, %d differing groups (near ties)" % (label, gm.shape[0], len(groups)))


def test_segment_offsets_bit_exact():
    rng = np.random.default_rng(1)
    for BH, N, G in [(3, 1000, 7), (2, 75600, 64), (1, 5, 1), (4, 3000, 300)]:
        labels = rng.integers(-1, G + 1, size=(BH, N)).astype(np.int32)
        _log("case segment offsets BH=%d N=%d G=%d" % (BH, N, G))
        got = api.segment_offsets(_gpu(labels), G).cpu().numpy()
        np.testing.assert_array_equal(got, oracle.segment_offsets(labels, G))


@pytest.mark.parametrize("d", [64, 128])
def test_segment_means_match_oracle(d):
    rng = np.random.default_rng(d)
    B, H, N, G = 2, 3, 1700, 9
    x = synth.f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32))
    labels = rng.integers(0, G, size=(B * H, N)).astype(np.int32)
    labels[1] = np.where(labels[1] == 4, 5, labels[1])            # an empty segment
    _log("case segment means d=%d" % d)
    perm = oracle.perm_from_labels(labels, G)
    xs = np.stack([x.reshape(B * H, N, d)[i][perm[i]] for i in range(B * H)]).reshape(B, H, N, d)
    ref = oracle.segment_means(xs, oracle.segment_offsets(labels, G))
    dx = _gpu(x.view(np.int16))
    gperm = api.perm_from_labels(_gpu(labels), G)
    gx = api.permute_rows(dx, gperm)
    got = api.segment_means(gx, api.segment_offsets(_gpu(labels), G)).cpu().numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=2e-6)
    assert np.all(got[1, 4] == 0)
    ref_t = oracle.segment_means(x, None, seg_len=128)
    got_t = api.segment_means(dx, seg_len=128).cpu().numpy()
    np.testing.assert_allclose(got_t, ref_t, rtol=1e-5, atol=2e-6)


@pytest.mark.parametrize("B,Hq,Hkv,N,block,d,G,m_exact,m_sample,spread", [
    (1, 2, 2, 1500, 64, 16, 5, 3, 6, 1.0),
    (2, 4, 2, 75600 // 4, 128, 128, 16, 8, 8, 0.8),
    (1, 3, 1, 4000, 64, 64, 7, 0, 12, 2.5),
    (1, 2, 2, 1000, 128, 32, 3, 5, 9, 1.0),          # residual no larger than the budget
    (1, 1, 1, 64 * 1024, 64, 8, 4, 16, 40, 0.5),     # 1024 tiles
    (1, 2, 2, 3000, 64, 24, 4, 4, 0, 1.0),           # exact set only
    (1, 2, 1, 20000, 64, 64, 6, 30, 50, 1.5),        # m_exact + m_sample > 64: every tile ranked by count
    (1, 2, 2, 9000, 64, 32, 5, 64, 0, 1.0),          # 64 exact tiles, the largest budget of the argmax rounds
])
def test_is_sample_matches_oracle(B, Hq, Hkv, N, block, d, G, m_exact, m_sample, spread):
    qbar, kbar, seg, uoff = _problem(N + G, B, Hq, Hkv, N, block, d, G, spread)
    _log("case is_sample B=%d Hq=%d Hkv=%d N=%d block=%d d=%d G=%d E=%d S=%d"
         % (B, Hq, Hkv, N, block, d, G, m_exact, m_sample))
    ref = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, m_sample)
    gm, glw, gpi = api.is_sample(_gpu(qbar), _gpu(kbar), _gpu(seg), _gpu(uoff), B, Hq, Hkv, N, block, m_exact,
                                 m_sample, want_pi=True)
    got = (gm.cpu().numpy(), glw.cpu().numpy(), gpi.cpu().numpy())
    _compare_sampler((qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, m_sample), got, ref, "random")


def test_is_sample_full_size():
    """Wan2.1-14B shape (40 heads x 75600 tokens, 64 clusters, 591 tiles,
    8 exact + 8 sampled tiles): oracle centroids of the clustered workload's
    permuted Q and K feed both sides."""
    t0 = time.time()
    w = synth.clustered(seed=4)
    _log("case is_sample full size (generated in %.1fs)" % (time.time() - t0))
    B, Hq, Hkv, N, block, C = w.B, w.Hq, w.Hkv, w.N, w.block, w.n_clusters
    pq = oracle.perm_from_labels(w.labels_q, C)
    pk = oracle.perm_from_labels(w.labels_k, C)
    qs = np.stack([w.q[0, h][pq[h]] for h in range(Hq)])[None]
    ks = np.stack([w.k[0, h][pk[h]] for h in range(Hkv)])[None]
    seg = oracle.segment_offsets(w.labels_q, C)
    qbar = oracle.segment_means(qs, seg)
    kbar = oracle.segment_means(ks, None, seg_len=block)
    uoff = np.random.default_rng(44).random((B * Hq, C))
    ref = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, 8, 8)
    gm, glw, gpi = api.is_sample(_gpu(qbar), _gpu(kbar), _gpu(seg), _gpu(uoff), B, Hq, Hkv, N, block, 8, 8,
                                 want_pi=True)
    got = (gm.cpu().numpy(), glw.cpu().numpy(), gpi.cpu().numpy())
    _compare_sampler((qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, 8, 8), got, ref, "full size")
    # the device centroids of the same inputs agree with the oracle's
    gq = api.permute_rows(_gpu(w.q.view(np.int16)), _gpu(pq))
    gk = api.permute_rows(_gpu(w.k.view(np.int16)), _gpu(pk))
    np.testing.assert_allclose(api.segment_means(gq, _gpu(seg)).cpu().numpy(), qbar, rtol=1e-5, atol=2e-6)
    np.testing.assert_allclose(api.segment_means(gk, seg_len=block).cpu().numpy(), kbar, rtol=1e-5, atol=2e-6)


@pytest.mark.parametrize("block,d,Hq,Hkv", [(128, 128, 2, 2), (64, 64, 4, 2)])
def test_sampled_pipeline_end_to_end(block, d, Hq, Hkv):
    w = synth.random_case(70 + block, B=1, Hq=Hq, Hkv=Hkv, N=block * 23 - 29, d=d, block=block, density=0.3,
                          permute=True, n_clusters=6)
    # one label set per query head and per KV head, as the workload gives
    C = w.n_clusters
    uoff = np.random.default_rng(block).random((w.B * w.Hq, C))
    E, S = 3, 4
    _log("case sampled pipeline block=%d d=%d Hq=%d Hkv=%d" % (block, d, Hq, Hkv))
    dw = pipeline.to_device(w)
    res = pipeline.forward(dw, want_lse=True, sampler={"m_exact": E, "m_sample": S, "uoff": _gpu(uoff)})
    torch.cuda.synchronize()
    # the oracle chain
    pq = oracle.perm_from_labels(w.labels_q, C)
    pk = oracle.perm_from_labels(w.labels_k, C)
    qs = np.stack([w.q[0, h][pq[h]] for h in range(Hq)])[None]
    ks = np.stack([w.k[0, h][pk[h]] for h in range(Hkv)])[None]
    seg = oracle.segment_offsets(w.labels_q, C)
    qbar = oracle.segment_means(qs, seg)
    kbar = oracle.segment_means(ks, None, seg_len=block)
    om, olw, _ = oracle.is_sample(qbar, kbar, seg, uoff, w.B, Hq, Hkv, w.N, block, E, S)
    rp, col, lw = oracle.build_csr(om, None, 0.0, olw, w.nQB, True)
    np.testing.assert_array_equal(res.row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(res.col.cpu().numpy(), col)
    np.testing.assert_allclose(res.lw.cpu().numpy(), lw, rtol=0, atol=1e-6)
    rows = sample_rows(w, seed=2)
    stats = compare_rows(w, res, rows, pq, pk, (rp, col, lw))
    _log("  %s" % stats)
    assert_within(stats)
