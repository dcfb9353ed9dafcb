"""Pins of the oracle's centroid and importance-sampling routines (InstaGen,
Algorithm 1 steps 2-13; section 3.2.1 Eq. 4 and the systematic PPS sample of
section 4).

* segment offsets / means: numpy bincount, stable argsort and mean (library
  routines).
* exact set: numpy lexsort of masses that numpy computes itself (matmul, exp).
* inclusion probabilities: scipy's brentq root of sum(min(1, lam s)) = m.
* systematic PPS: over a grid of offsets the empirical inclusion frequency
  of every tile is its probability, and every sample has exactly m tiles
  (exact properties of systematic sampling; grid error at most 1/grid).
* Horvitz-Thompson: the weighted estimate of a sum is unbiased over the grid.
* special cases: equal masses give the UNIFORM sampler's m/|R| (Algorithm 1
  step 7), a dominant tile is promoted (pi = 1, weight 1), a residual no
  larger than the budget is kept whole, GQA reads the shared key head.
"""
import numpy as np
import pytest
from scipy.optimize import brentq

import oracle
import synth


def problem(seed, B=1, Hq=2, Hkv=2, N=1000, block=64, d=16, G=5, spread=1.0):
    rng = np.random.default_rng(seed)
    nb = -(-N // block)
    qbar = (rng.standard_normal((B * Hq, G, d)) * spread).astype(np.float32)
    kbar = (rng.standard_normal((B * Hkv, nb, d)) * spread).astype(np.float32)
    labels = rng.integers(0, G, size=(B * Hq, N)).astype(np.int32)
    seg = oracle.segment_offsets(labels, G)
    uoff = rng.random((B * Hq, G))
    return qbar, kbar, seg, uoff


def masses(qbar, kbar, B, Hq, Hkv, N, block):
    d = qbar.shape[2]
    nb = kbar.shape[1]
    size = np.minimum(block, N - np.arange(nb) * block).astype(np.float64)
    out = np.empty((B * Hq, qbar.shape[1], nb))
    for bh in range(B * Hq):
        b, h = divmod(bh, Hq)
        a = (qbar[bh].astype(np.float64) @ kbar[b * Hkv + h // (Hq // Hkv)].astype(np.float64).T) / np.sqrt(d)
        out[bh] = size[None, :] * np.exp(a - a.max(1, keepdims=True))
    return out


def group_rows(seg, g, block, nb):
    u0 = -(-int(seg[g]) // block)
    u1 = min(nb, -(-int(seg[g + 1]) // block))
    return range(u0, u1)


def test_segment_offsets_matches_bincount():
    rng = np.random.default_rng(1)
    labels = rng.integers(-2, 9, size=(3, 500)).astype(np.int32)
    sp = oracle.segment_offsets(labels, 7)
    for bh in range(3):
        ok = labels[bh][(labels[bh] >= 0) & (labels[bh] < 7)]
        counts = np.bincount(ok, minlength=7)
        np.testing.assert_array_equal(sp[bh], np.concatenate([[0], np.cumsum(counts)]))


def test_segment_means_match_numpy():
    rng = np.random.default_rng(2)
    B, H, N, d, G = 2, 3, 700, 24, 6
    x = synth.f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32))
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    labels = rng.integers(0, G, size=(B * H, N)).astype(np.int32)
    labels[0, :] = np.where(labels[0] == 3, 2, labels[0])          # an empty segment
    sp = oracle.segment_offsets(labels, G)
    perm = np.stack([np.argsort(labels[i], kind="stable") for i in range(B * H)])
    xs = np.stack([xf.reshape(B * H, N, d)[i][perm[i]] for i in range(B * H)]).reshape(B, H, N, d)
    xs_bits = synth.f32_to_bf16_bits(xs.astype(np.float32))
    got = oracle.segment_means(xs_bits, sp)
    for i in range(B * H):
        for g in range(G):
            rows = xf.reshape(B * H, N, d)[i][labels[i] == g]
            ref = rows.mean(0) if len(rows) else np.zeros(d)
            np.testing.assert_allclose(got[i, g], ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    assert np.all(got[0, 3] == 0)
    # fixed-length segments (tile means) with a partial last tile
    tiles = oracle.segment_means(x, None, seg_len=64)
    assert tiles.shape == (B * H, 11, d)
    for t in range(11):
        ref = xf.reshape(B * H, N, d)[:, t * 64:min(N, t * 64 + 64)].mean(1)
        np.testing.assert_allclose(tiles[:, t], ref.astype(np.float32), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("m_exact", [0, 1, 5, 16])
def test_exact_set_is_top_by_mass(m_exact):
    B, Hq, Hkv, N, block = 1, 3, 3, 1500, 64
    qbar, kbar, seg, uoff = problem(3 + m_exact, B, Hq, Hkv, N, block)
    nb = kbar.shape[1]
    mask, lw, pi = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, 0)
    M = masses(qbar, kbar, B, Hq, Hkv, N, block)
    for bh in range(B * Hq):
        for g in range(qbar.shape[1]):
            order = np.lexsort((np.arange(nb), -M[bh, g]))
            want = np.zeros(nb, bool)
            want[order[:m_exact]] = True
            for u in group_rows(seg[bh], g, block, nb):
                np.testing.assert_array_equal(mask[bh * nb + u] != 0, want)
                assert np.all(lw[bh * nb + u] == 0)


@pytest.mark.parametrize("m_sample,spread", [(4, 1.0), (8, 3.0), (12, 0.3)])
def test_inclusion_probabilities_solve_eq4(m_sample, spread):
    B, Hq, Hkv, N, block, m_exact = 1, 2, 1, 2000, 64, 3
    qbar, kbar, seg, uoff = problem(10 + m_sample, B, Hq, Hkv, N, block, spread=spread)
    nb = kbar.shape[1]
    _, _, pi = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, m_sample)
    M = masses(qbar, kbar, B, Hq, Hkv, N, block)
    for bh in range(B * Hq):
        for g in range(qbar.shape[1]):
            order = np.lexsort((np.arange(nb), -M[bh, g]))
            resid = np.sort(order[m_exact:])
            s = M[bh, g, resid]
            lam = brentq(lambda x: np.minimum(1.0, x * s).sum() - m_sample, 0.0, 1e6 / s.min(), xtol=1e-300,
                         rtol=1e-15)
            np.testing.assert_allclose(pi[bh, g, resid], np.minimum(1.0, lam * s), rtol=1e-10, atol=0)
            assert abs(pi[bh, g, resid].sum() - m_sample) < 1e-9
            assert np.all(pi[bh, g, order[:m_exact]] == 1.0)


def test_systematic_pps_hits_its_probabilities_exactly():
    B, Hq, Hkv, N, block, m_exact, m_sample = 1, 2, 2, 1200, 64, 2, 6
    qbar, kbar, seg, _ = problem(20, B, Hq, Hkv, N, block, G=3, spread=1.5)
    nb = kbar.shape[1]
    grid = 1024
    freq = np.zeros((B * Hq, 3, nb))
    y = np.random.default_rng(5).random(nb) + 0.1
    ht = np.zeros((B * Hq, 3))
    pi = None
    for i in range(grid):
        uoff = np.full((B * Hq, 3), (i + 0.5) / grid)
        mask, lw, pi = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, m_exact, m_sample)
        for bh in range(B * Hq):
            for g in range(3):
                rows = group_rows(seg[bh], g, block, nb)
                if len(rows) == 0:
                    continue
                kept = mask[bh * nb + rows[0]] != 0
                exact_or_promoted = pi[bh, g] == 1.0
                resid_kept = kept & (pi[bh, g] < 1.0)
                # every sample has m_exact + m_sample tiles
                assert kept.sum() == m_exact + m_sample
                freq[bh, g] += kept
                ht[bh, g] += (y[exact_or_promoted & kept]).sum() + (y[resid_kept] / pi[bh, g, resid_kept]).sum()
    for bh in range(B * Hq):
        for g in range(3):
            if len(group_rows(seg[bh], g, block, nb)) == 0:
                continue
            p = pi[bh, g]
            np.testing.assert_allclose(freq[bh, g] / grid, p, atol=1.0 / grid + 1e-12)
            bound = (y / np.maximum(p, 1e-300))[p < 1].sum() / grid + 1e-9
            assert abs(ht[bh, g] / grid - y.sum()) <= bound


def test_equal_masses_give_the_uniform_sampler():
    B, Hq, Hkv, N, block, d, G = 1, 1, 1, 64 * 40, 64, 8, 2
    rng = np.random.default_rng(7)
    qbar = rng.standard_normal((1, G, d)).astype(np.float32)
    kbar = np.tile(rng.standard_normal((1, 1, d)).astype(np.float32), (1, 40, 1))
    seg = np.array([[0, 1000, N]], np.int32)
    mask, lw, pi = oracle.is_sample(qbar, kbar, seg, np.array([[0.3, 0.9]]), B, Hq, Hkv, N, block, 4, 9)
    for g in range(G):
        assert np.all(pi[0, g, :4] == 1.0)                    # ties go to the lower tiles
        np.testing.assert_allclose(pi[0, g, 4:], 9 / 36, rtol=1e-14)
        u = group_rows(seg[0], g, block, 40)[0]
        kept = np.nonzero(mask[u])[0]
        assert len(kept) == 13
        sampled = kept[kept >= 4]
        np.testing.assert_allclose(lw[u, sampled[sampled != u]], np.float32(-np.log(9 / 36)), rtol=1e-7)


def test_dominant_tile_is_promoted():
    B, Hq, Hkv, N, block, d = 1, 1, 1, 64 * 30, 64, 8
    rng = np.random.default_rng(8)
    qbar = rng.standard_normal((1, 1, d)).astype(np.float32)
    kbar = (rng.standard_normal((1, 30, d)) * 0.1).astype(np.float32)
    kbar[0, 17] = qbar[0, 0] * 8.0                             # mass far above the rest
    seg = np.array([[0, N]], np.int32)
    mask, lw, pi = oracle.is_sample(qbar, kbar, seg, np.array([[0.5]]), B, Hq, Hkv, N, block, 0, 5)
    assert pi[0, 0, 17] == 1.0
    others = np.delete(pi[0, 0], 17)
    assert np.all(others < 1.0)
    assert abs(others.sum() - 4.0) < 1e-12
    assert np.all(mask[:, 17] == 1) and np.all(lw[:, 17] == 0)


def test_small_residual_is_kept_whole_and_rows_follow_groups():
    B, Hq, Hkv, N, block = 1, 2, 2, 640, 64                   # 10 tiles
    qbar, kbar, seg, uoff = problem(30, B, Hq, Hkv, N, block, G=4)
    seg[1, 4] = 500                                            # tokens 500.. of head 1 have no group
    seg[1] = np.minimum(seg[1], 500)
    mask, lw, pi = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, 3, 7)
    nb = 10
    for bh in range(2):
        covered = np.zeros(nb, bool)
        for g in range(4):
            for u in group_rows(seg[bh], g, block, nb):
                covered[u] = True
                assert np.all(mask[bh * nb + u] == 1)
                assert np.all(lw[bh * nb + u] == 0)
        for u in np.nonzero(~covered)[0]:
            assert np.all(mask[bh * nb + u] == 0)
    assert not np.all(mask[nb + 8:] == 1)                      # head 1, blocks 8..9 have no group


def test_gqa_reads_the_shared_key_head():
    B, Hq, Hkv, N, block = 1, 4, 2, 1100, 64
    qbar, kbar, seg, uoff = problem(40, B, Hq, Hkv, N, block)
    m1 = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, 3, 5)
    kfull = np.repeat(kbar, 2, axis=0)                         # query head h -> key head h // 2
    m2 = oracle.is_sample(qbar, kfull, seg, uoff, B, Hq, Hq, N, block, 3, 5)
    for a, b in zip(m1, m2):
        np.testing.assert_array_equal(a, b)


def test_lw_is_minus_log_pi_and_diagonal_is_exact():
    B, Hq, Hkv, N, block = 1, 2, 2, 3000, 64
    qbar, kbar, seg, uoff = problem(50, B, Hq, Hkv, N, block, G=3, spread=0.7)
    nb = kbar.shape[1]
    mask, lw, pi = oracle.is_sample(qbar, kbar, seg, uoff, B, Hq, Hkv, N, block, 4, 10)
    for bh in range(B * Hq):
        for g in range(3):
            for u in group_rows(seg[bh], g, block, nb):
                r = bh * nb + u
                kept = np.nonzero(mask[r])[0]
                for v in kept:
                    want = 0.0 if (pi[bh, g, v] == 1.0 or v == u) else -np.log(pi[bh, g, v])
                    assert lw[r, v] == np.float32(want)
                assert np.all(lw[r][mask[r] == 0] == 0)
