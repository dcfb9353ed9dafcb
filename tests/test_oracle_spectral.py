"""Pins of the oracle's WaveAlign stage-1 row order (polar angle of a rank-2
embedding of the centred mask rows, WaveAlign section IV-C).

* numpy's SVD of the dense centred mask (library routine): after enough
  iterations every row's angle equals +-(its angle in the top-2 left singular
  vectors) + one constant, i.e. the same subspace up to a rotation or
  reflection of the plane, which the order does not see.
* closed form: for a circulant band mask the top-2 centred singular vectors
  are the first Fourier pair, so the order is a rotation (or reversal) of the
  rows.
* invariants: identical rows sit together in index order; permuting the KV
  columns or adding a block every row lists leaves the angles unchanged
  (centring removes the constant column).
"""
import numpy as np
import pytest

import oracle


def csr_from_dense(m):
    rows, cols = np.nonzero(m)
    rp = np.concatenate([[0], np.cumsum(m.sum(1))]).astype(np.int32)
    return rp, cols.astype(np.int32)


def planted_mask(rng, n, nk, density=0.2):
    """Rows drawn around three prototype rows: after centring, two large
    singular values and a noise floor."""
    protos = rng.random((3, nk)) < density
    lab = rng.integers(0, 3, size=n)
    m = protos[lab].copy()
    flip = rng.random((n, nk)) < 0.02
    return (m ^ flip).astype(np.uint8)


def wrap(d):
    return (d + np.pi) % (2 * np.pi) - np.pi


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_angles_match_numpy_svd(seed):
    rng = np.random.default_rng(seed)
    n, nk = 120, 90
    m = planted_mask(rng, n, nk)
    rp, col = csr_from_dense(m)
    perm, ang = oracle.spectral_order(rp, col, 1, n, nk, 400)
    c = m.astype(np.float64) - m.mean(0, keepdims=True)
    u, s, _ = np.linalg.svd(c, full_matrices=False)
    assert s[1] > 1.5 * s[2]                       # a well separated top-2 subspace
    phi = np.arctan2(u[:, 1], u[:, 0])
    r = np.hypot(u[:, 0], u[:, 1])
    big = r > 1e-3 * r.max()
    ok = False
    for sign in (1.0, -1.0):
        d = wrap(ang[0] - sign * phi)[big]
        ok |= np.abs(wrap(d - d[0])).max() < 1e-6
    assert ok
    # the order is ascending in angle, ties by index
    a = ang[0][perm[0]]
    assert np.all(np.diff(a) >= 0)
    assert sorted(perm[0].tolist()) == list(range(n))


@pytest.mark.parametrize("n,w", [(64, 5), (100, 11)])
def test_circulant_band_orders_rows_around_the_circle(n, w):
    m = np.zeros((n, n), np.uint8)
    for i in range(n):
        for k in range(-w, w + 1):
            m[i, (i + k) % n] = 1
    rp, col = csr_from_dense(m)
    perm, ang = oracle.spectral_order(rp, col, 1, n, n, 200)
    p = perm[0]
    # consecutive positions hold circularly adjacent rows, one direction throughout
    steps = (np.diff(np.concatenate([p, p[:1]])) % n)
    assert np.all(steps == 1) or np.all(steps == n - 1)


def test_identical_rows_are_adjacent_in_index_order():
    rng = np.random.default_rng(5)
    n, nk = 90, 70
    protos = (rng.random((6, nk)) < 0.25).astype(np.uint8)
    lab = rng.integers(0, 6, size=n)
    m = protos[lab]
    rp, col = csr_from_dense(m)
    perm, ang = oracle.spectral_order(rp, col, 1, n, nk, 30)
    p = perm[0]
    for g in range(6):
        pos = np.nonzero(lab[p] == g)[0]
        if len(pos):
            assert pos.max() - pos.min() + 1 == len(pos)        # contiguous
            assert np.all(np.diff(p[pos]) > 0)                   # ascending index
            assert np.ptp(ang[0][lab == g]) == 0.0


def test_column_permutation_and_constant_column_leave_angles():
    rng = np.random.default_rng(7)
    n, nk = 80, 60
    m = planted_mask(rng, n, nk, 0.3)
    rp, col = csr_from_dense(m)
    _, a0 = oracle.spectral_order(rp, col, 1, n, nk, 60)
    cp = rng.permutation(nk)
    m1 = m[:, cp]
    rp1, col1 = csr_from_dense(m1)
    _, a1 = oracle.spectral_order(rp1, col1, 1, n, nk, 60)
    np.testing.assert_allclose(a1, a0, atol=1e-9)
    m2 = np.concatenate([m, np.ones((n, 1), np.uint8)], 1)
    rp2, col2 = csr_from_dense(m2)
    _, a2 = oracle.spectral_order(rp2, col2, 1, n, nk + 1, 60)
    np.testing.assert_allclose(a2, a0, atol=1e-9)


def test_heads_are_independent():
    rng = np.random.default_rng(9)
    n, nk = 50, 40
    ms = [planted_mask(rng, n, nk) for _ in range(3)]
    rp_all, col_all = csr_from_dense(np.concatenate(ms, 0))
    perm, ang = oracle.spectral_order(rp_all, col_all, 3, n, nk, 25)
    for h in range(3):
        rp, col = csr_from_dense(ms[h])
        p1, a1 = oracle.spectral_order(rp, col, 1, n, nk, 25)
        np.testing.assert_array_equal(perm[h], p1[0])
        np.testing.assert_array_equal(ang[h], a1[0])
