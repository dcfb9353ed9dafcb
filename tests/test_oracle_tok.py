"""Pins of the oracle's token-level attention over computational query sets
(INTRA, sections 3 and 4.8; InstaGen Eq. (1)-(3) over each set's key list)
and of the query-set index maps.

* torch CPU fp64 scaled_dot_product_attention on the gathered query and key
  rows (library routine), with causal and out-of-range entries masked and
  duplicate entries kept as separate terms.
* Block-shaped sets (a query block attending to every token of its listed
  KV blocks) reproduce the block-sparse oracle, which has pins of its own.
* Closed forms: constant V gives that constant; an empty list gives O = 0,
  LSE = -inf; an empty slot gives NaN.
* Index maps: INTRA Scatter covers every token once and lists each group's
  members; Gather 1 (cyclic segments) covers every token once, lists whole
  segments, and meets every Scatter group in exactly T / R tokens; Gather 0
  lists 256 distinct in-image keys per patch, in four tiles of four rows of
  16, containing the patch, shifted inward at edges.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def rand_qkv(seed, B, Hq, Hkv, N, d):
    g = np.random.default_rng(seed)
    f = lambda H: synth.f32_to_bf16_bits(g.standard_normal((B, H, N, d)).astype(np.float32))
    return f(Hq), f(Hkv), f(Hkv)


def sdpa_ref(q, k, v, q_idx, kv_ptr, kv_idx, causal):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    C, BQ = q_idx.shape[1], q_idx.shape[2]
    qf, kf, vf = (torch.from_numpy(synth.bf16_bits_to_f32(x).astype(np.float64)) for x in (q, k, v))
    outs, lses = [], []
    for bh in range(B * Hq):
        b, h = divmod(bh, Hq)
        g = h // (Hq // Hkv)
        for c in range(C):
            cq = bh * C + c
            keys = kv_idx[kv_ptr[cq]:kv_ptr[cq + 1]].astype(np.int64)
            for t in q_idx[bh, c]:
                if t < 0 or t >= N:
                    outs.append(np.zeros(d))
                    lses.append(np.nan)
                    continue
                ok = (keys >= 0) & (keys < N)
                if causal:
                    ok &= keys <= t
                if not ok.any():
                    outs.append(np.zeros(d))
                    lses.append(-np.inf)
                    continue
                kk = torch.from_numpy(np.clip(keys, 0, N - 1))
                K = kf[b, g][kk]
                V = vf[b, g][kk]
                mask = torch.from_numpy(np.where(ok, 0.0, -np.inf))
                Q = qf[b, h][int(t)][None]
                o = torch.nn.functional.scaled_dot_product_attention(Q[None], K[None], V[None],
                                                                     attn_mask=mask[None, None])[0, 0]
                x = (K @ Q[0]) / np.sqrt(d) + mask
                outs.append(o.numpy())
                lses.append(float(torch.logsumexp(x, 0)))
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa(causal):
    B, Hq, Hkv, N, d, C, BQ = 1, 4, 2, 300, 16, 5, 8
    q, k, v = rand_qkv(11 + causal, B, Hq, Hkv, N, d)
    g = np.random.default_rng(5)
    q_idx = g.integers(-3, N + 3, size=(B * Hq, C, BQ)).astype(np.int32)
    lens = g.integers(0, 70, size=B * Hq * C)
    lens[3] = 0
    kv_ptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kv_idx = g.integers(-2, N + 2, size=int(kv_ptr[-1])).astype(np.int32)
    kv_idx[5] = kv_idx[6]                                   # a duplicate entry: two terms
    out, lse = oracle.attn_tok(q, k, v, q_idx, kv_ptr, kv_idx, causal=causal)
    ro, rl = sdpa_ref(q, k, v, q_idx, kv_ptr, kv_idx, causal)
    np.testing.assert_allclose(out, ro, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isnan(lse), np.isnan(rl))
    fin = np.isfinite(rl)
    np.testing.assert_allclose(lse[fin], rl[fin], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(lse[np.isneginf(rl)]))


def test_block_shaped_sets_match_block_sparse_oracle():
    B, Hq, Hkv, N, d, block = 1, 2, 1, 200, 16, 32
    w = synth.random_case(17, B=B, Hq=Hq, Hkv=Hkv, N=N, d=d, block=block, density=0.4)
    rp, col, _ = oracle.build_csr(w.mask, None, 0.0, None, w.nQB, True)
    nb = w.nQB
    q_idx = np.full((B * Hq, nb, block), -1, np.int32)
    lists = []
    for bh in range(B * Hq):
        for u in range(nb):
            t = np.arange(u * block, min(N, (u + 1) * block))
            q_idx[bh, u, :len(t)] = t
            r = bh * nb + u
            lists.append(np.concatenate([np.arange(c * block, min(N, (c + 1) * block)) for c in col[rp[r]:rp[r + 1]]]))
    kv_ptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    kv_idx = np.concatenate(lists).astype(np.int32)
    for causal in (False, True):
        out, lse = oracle.attn_tok(w.q, w.k, w.v, q_idx, kv_ptr, kv_idx, causal=causal)
        ok = q_idx.reshape(-1) >= 0
        rows = np.array([bh * N + t for bh in range(B * Hq) for t in q_idx[bh].reshape(-1) if t >= 0], np.int64)
        ro, rl = oracle.attn_rows(w.q, w.k, w.v, rp, col, None, block, rows, causal=causal)
        np.testing.assert_allclose(out[ok], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[ok], rl, rtol=0, atol=1e-12)


def test_constant_values_and_empty_lists():
    B, Hq, Hkv, N, d = 1, 1, 1, 64, 8
    q, k, _ = rand_qkv(3, B, Hq, Hkv, N, d)
    v = np.full((B, Hkv, N, d), synth.f32_to_bf16_bits(np.array([0.75], np.float32))[0], np.uint16)
    q_idx = np.array([[[0, 5, -1, 70], [10, 11, 12, 13]]], np.int32)
    kv_ptr = np.array([0, 3, 3], np.int32)
    kv_idx = np.array([4, 9, 60], np.int32)
    out, lse = oracle.attn_tok(q, k, v, q_idx, kv_ptr, kv_idx)
    np.testing.assert_allclose(out[:2], 0.75, rtol=0, atol=1e-15)
    assert np.isnan(lse[2]) and np.isnan(lse[3]) and np.all(out[2:4] == 0)
    assert np.all(out[4:] == 0) and np.all(np.isneginf(lse[4:]))


def test_scatter_map_covers_every_token_once():
    for N, R, causal in [(1000, 8, False), (4096, 8, True), (777, 4, True)]:
        q_idx, kv_ptr, kv_idx = synth.cqs_scatter(N, R, 64, causal)
        qs = q_idx[q_idx >= 0]
        np.testing.assert_array_equal(np.sort(qs), np.arange(N))
        for c in range(q_idx.shape[0]):
            keys = kv_idx[kv_ptr[c]:kv_ptr[c + 1]]
            qc = q_idx[c][q_idx[c] >= 0]
            r = qc[0] % R
            assert np.all(keys % R == r) and np.all(qc % R == r)
            members = np.arange(r, N, R)
            want = members[members <= qc.max()] if causal else members
            np.testing.assert_array_equal(keys, want)


@pytest.mark.parametrize("N,R,causal", [(4096, 8, False), (4096, 8, True), (1000, 8, True), (777, 4, False)])
def test_gather1_map_is_cyclic_segments(N, R, causal):
    q_idx, kv_ptr, kv_idx = synth.cqs_gather1(N, R, 64, causal)
    qs = q_idx[q_idx >= 0]
    np.testing.assert_array_equal(np.sort(qs), np.arange(N))          # every token in exactly one set
    for c in range(q_idx.shape[0]):
        qc = q_idx[c][q_idx[c] >= 0]
        b = (qc[0] // R) % R
        assert np.all((qc // R) % R == b)                              # one group per set
        members = np.array([t for t in range(N) if (t // R) % R == b])
        keys = kv_idx[kv_ptr[c]:kv_ptr[c + 1]]
        np.testing.assert_array_equal(keys, members[members <= qc.max()] if causal else members)
    # the relay property of the cyclic Gather: with N = T R and T a multiple
    # of R, every Gather group shares exactly T / R tokens with every Scatter
    # group (local index t mod R)
    if N % (R * R) == 0:
        T = N // R
        groups = [np.array([t for t in range(N) if (t // R) % R == b]) for b in range(R)]
        for b in range(R):
            for r in range(R):
                assert np.sum(groups[b] % R == r) == T // R


@pytest.mark.parametrize("H,W", [(16, 16), (32, 48), (64, 64)])
def test_gather0_windows(H, W):
    q_idx, kv_ptr, kv_idx = synth.cqs_gather0(H, W)
    assert q_idx.shape == ((H // 8) * (W // 8), 64)
    np.testing.assert_array_equal(np.sort(q_idx.reshape(-1)), np.arange(H * W))
    for i in range(q_idx.shape[0]):
        keys = kv_idx[kv_ptr[i]:kv_ptr[i + 1]]
        assert len(keys) == 256 and len(np.unique(keys)) == 256
        assert keys.min() >= 0 and keys.max() < H * W
        rows, cols = keys // W, keys % W
        assert rows.max() - rows.min() == 15 and cols.max() - cols.min() == 15
        assert set(q_idx[i]) <= set(keys)                     # the window contains its patch
        for t in range(4):                                    # tile t: rows 4t..4t+3 of the window
            tile = keys[64 * t:64 * t + 64]
            assert len(np.unique(tile // W)) == 4
        r, c = divmod(i, W // 8)
        assert rows.min() == min(max(8 * r - 4, 0), H - 16)
        assert cols.min() == min(max(8 * c - 4, 0), W - 16)
