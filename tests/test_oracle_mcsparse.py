"""Pins of the oracle's exact token selection (MC-Sparse, implementation
details: a dense first pass for each query's log-sum-exp; a second pass that
recovers the attention probabilities, sums them per query group and takes
the top-K keys by that mass).

* brute force on tiny inputs: pure-Python loops with math.exp;
* closed form: every query's probabilities sum to 1, so a group's masses sum
  to its number of valid queries (empty slots add nothing);
* causal: no mass after the group's last query;
* closed form: with every key equal, each probability is 1/N (causal:
  1/(t+1) on the keys up to t);
* a restricted key range is the slice of the full result;
* top-K: numpy's lexsort by (mass descending, index ascending), with planted
  ties, K >= N and K = 0.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def qk(seed, B, Hq, Hkv, N, d, scale=1.0):
    g = np.random.default_rng(seed)
    f = lambda H: synth.f32_to_bf16_bits((g.standard_normal((B, H, N, d)) * scale).astype(np.float32))
    return f(Hq), f(Hkv)


def brute_mass(q, k, q_idx, causal):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    C, BQ = q_idx.shape[1], q_idx.shape[2]
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    kf = synth.bf16_bits_to_f32(k).astype(np.float64)
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((B * Hq * C, N))
    for bh in range(B * Hq):
        b, h = divmod(bh, Hq)
        g = h // (Hq // Hkv)
        for c in range(C):
            for t in q_idx[bh, c]:
                if t < 0 or t >= N:
                    continue
                keys = range(t + 1) if causal else range(N)
                x = [scale * sum(qf[b, h, t, i] * kf[b, g, s, i] for i in range(d)) for s in keys]
                m = max(x)
                lse = m + math.log(sum(math.exp(v - m) for v in x))
                for s, v in zip(keys, x):
                    out[bh * C + c, s] += math.exp(v - lse)
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_group_mass_matches_brute_force(causal):
    B, Hq, Hkv, N, d, C, BQ = 2, 4, 2, 40, 8, 3, 8       # two query heads share each KV head
    q, k = qk(3 + causal, B, Hq, Hkv, N, d, scale=2.0)
    g = np.random.default_rng(9)
    q_idx = g.integers(-2, N + 2, size=(B * Hq, C, BQ)).astype(np.int32)
    got = oracle.group_mass(q, k, q_idx, causal=causal)
    np.testing.assert_allclose(got, brute_mass(q, k, q_idx, causal), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_group_mass_sums_to_query_count(causal):
    B, Hq, Hkv, N, d, C, BQ = 1, 4, 2, 300, 16, 5, 32
    q, k = qk(5, B, Hq, Hkv, N, d, scale=3.0)
    g = np.random.default_rng(10)
    q_idx = g.integers(-5, N, size=(B * Hq, C, BQ)).astype(np.int32)
    mass = oracle.group_mass(q, k, q_idx, causal=causal)
    count = ((q_idx >= 0) & (q_idx < N)).sum(axis=2).reshape(-1)
    np.testing.assert_allclose(mass.sum(axis=1), count, rtol=0, atol=1e-12)
    assert np.all(mass >= 0)
    if causal:
        for r in range(mass.shape[0]):
            qs = q_idx.reshape(-1, BQ)[r]
            qs = qs[(qs >= 0) & (qs < N)]
            last = qs.max() if len(qs) else -1
            assert np.all(mass[r, last + 1:] == 0)


def test_key_range_is_a_slice():
    B, Hq, Hkv, N, d, C, BQ = 1, 2, 2, 200, 16, 3, 16
    q, k = qk(6, B, Hq, Hkv, N, d)
    q_idx = np.random.default_rng(11).integers(0, N, size=(B * Hq, C, BQ)).astype(np.int32)
    full = oracle.group_mass(q, k, q_idx)
    part = oracle.group_mass(q, k, q_idx, keys=(37, 151))
    np.testing.assert_array_equal(part, full[:, 37:151])


def lexsort_topk(mass, K):
    rows, N = mass.shape
    out = []
    for r in range(rows):
        order = np.lexsort((np.arange(N), -mass[r]))   # mass descending, then index ascending
        out.append(np.sort(order[:min(K, N)]))
    return np.array(out, dtype=np.int32).reshape(rows, min(K, N))


@pytest.mark.parametrize("K", [0, 1, 7, 64, 300, 1000])
def test_topk_matches_lexsort_with_ties(K):
    g = np.random.default_rng(12)
    rows, N = 6, 300
    mass = g.random((rows, N)).astype(np.float32)
    mass[1] = 0.5                                        # one row of equal masses
    mass[2, ::3] = mass[2, 5]                            # a block of ties at one value
    mass[3, :] = np.round(mass[3] * 4) / 4               # few distinct values
    mass[4, 10:20] = 0.0
    got = oracle.topk(mass, K)
    np.testing.assert_array_equal(got, lexsort_topk(mass.astype(np.float64), K))
    assert got.shape == (rows, min(K, N))
    if K > 0:
        assert np.all(np.diff(got, axis=1) > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_group_mass_closed_form_equal_keys(causal):
    """Every key the same vector: each query's scores are all equal, so its
    probabilities are 1/N (causal: 1/(t+1) on keys s <= t) and a key's mass is
    the sum of those over the group's queries."""
    B, Hq, Hkv, N, d, C, BQ = 1, 2, 1, 97, 16, 4, 8
    g = np.random.default_rng(14)
    q = synth.f32_to_bf16_bits(g.standard_normal((B, Hq, N, d)).astype(np.float32))
    row = synth.f32_to_bf16_bits(g.standard_normal(d).astype(np.float32))
    k = np.broadcast_to(row, (B, Hkv, N, d)).copy()
    q_idx = g.integers(-3, N, size=(B * Hq, C, BQ)).astype(np.int32)
    got = oracle.group_mass(q, k, q_idx, causal=causal)
    want = np.zeros_like(got)
    for r, ts in enumerate(q_idx.reshape(-1, BQ)):
        for t in ts[(ts >= 0) & (ts < N)]:
            if causal:
                want[r, :t + 1] += 1.0 / (t + 1)
            else:
                want[r] += 1.0 / N
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-15)
