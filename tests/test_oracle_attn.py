"""Pins of the CPU oracle's attention against things other than itself.

* library routine: torch's CPU fp64 scaled_dot_product_attention, with a dense
  boolean or additive mask built straight from the block mask (never from the
  oracle's CSR), in permuted token space when there is a permutation;
* brute force on tiny inputs (pure Python loops, Eq. 2 of InstaGen section 3.1
  without max subtraction);
* closed forms and invariants: constant V, Q = 0 (weighted block mean),
  log-weight shift, the Horvitz-Thompson identity that a log-weight of ln 2
  on a block equals duplicating that block's keys and values (InstaGen,
  section 4, the estimators of n_i and z_i), empty rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

torch.set_default_dtype(torch.float64)


def f64(bits):
    return torch.from_numpy(synth.bf16_bits_to_f32(bits).astype(np.float64))


def dense_token_bias(w, perm_q, perm_k):
    """Additive [B*Hq][N][N] bias in *permuted* token space from the block mask
    (or T <= p), the forced diagonal and the log-weight map: 0/lw where
    allowed, -inf elsewhere."""
    nb = w.nQB
    src = (w.mask != 0) if w.mask is not None else (w.T <= np.float32(w.p))
    keep = src.reshape(w.B * w.Hq, nb, nb).copy()
    if w.force_diag:
        keep[:, np.arange(nb), np.arange(nb)] = True
    lw = np.zeros_like(keep, dtype=np.float64) if w.lw_map is None else \
        w.lw_map.reshape(w.B * w.Hq, nb, nb).astype(np.float64)
    blk = np.arange(w.N) // w.block
    tok_keep = keep[:, blk][:, :, blk]
    tok_bias = np.where(tok_keep, lw[:, blk][:, :, blk], -np.inf)
    return torch.from_numpy(tok_bias)


def sdpa_reference(w, perm_q=None, perm_k=None):
    """O [B][Hq][N][d] in original token order via torch SDPA with a dense mask."""
    q, k, v = f64(w.q), f64(w.k), f64(w.v)
    G = w.Hq // w.Hkv
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    if perm_q is not None:
        pq = torch.from_numpy(perm_q.astype(np.int64)).view(w.B, w.Hq, w.N)
        pk = torch.from_numpy(perm_k.astype(np.int64)).view(w.B, w.Hkv, w.N).repeat_interleave(G, dim=1)
        q = torch.gather(q, 2, pq[..., None].expand_as(q))
        k = torch.gather(k, 2, pk[..., None].expand_as(k))
        v = torch.gather(v, 2, pk[..., None].expand_as(v))
    bias = dense_token_bias(w, perm_q, perm_k).view(w.B, w.Hq, w.N, w.N)
    if w.causal:
        assert perm_q is None
        bias = bias.masked_fill(torch.ones(w.N, w.N, dtype=torch.bool).triu(1), -math.inf)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=bias)
    if perm_q is not None:
        out = torch.empty_like(o)
        out.scatter_(2, pq[..., None].expand_as(o), o)
        o = out
    return o.numpy()


def oracle_all(w):
    perm_q = perm_k = None
    if w.permuted:
        perm_q = oracle.perm_from_labels(w.labels_q, w.n_clusters)
        perm_k = oracle.perm_from_labels(w.labels_k, w.n_clusters)
    rp, col, lw = oracle.build_csr(w.mask, w.T, w.p, w.lw_map, w.nQB, w.force_diag)
    O, L = oracle.attn_full(w, rp, col, lw, perm_q, perm_k)
    return O.reshape(w.B, w.Hq, w.N, w.d), L.reshape(w.B, w.Hq, w.N), perm_q, perm_k


CASES = [
    dict(B=1, Hq=2, Hkv=2, N=256, d=16, block=32, density=1.1),                    # full mask
    dict(B=2, Hq=3, Hkv=3, N=200, d=16, block=32, density=0.3),                    # ragged tail
    dict(B=1, Hq=4, Hkv=2, N=150, d=8, block=16, density=0.4, log_weights=True),   # GQA + lw
    dict(B=1, Hq=2, Hkv=1, N=130, d=8, block=16, density=0.5, causal=True),        # causal GQA
    dict(B=2, Hq=2, Hkv=2, N=190, d=8, block=32, density=0.35, permute=True, log_weights=True),
    dict(B=1, Hq=2, Hkv=2, N=160, d=16, block=16, density=0.25, use_T=True, permute=True),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_oracle_matches_sdpa_dense_mask(ci):
    w = synth.random_case(100 + ci, **CASES[ci])
    O, _, pq, pk = oracle_all(w)
    ref = sdpa_reference(w, pq, pk)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_oracle_full_mask_is_plain_sdpa():
    w = synth.random_case(7, B=1, Hq=2, Hkv=2, N=96, d=16, block=32, density=2.0)
    O, L, _, _ = oracle_all(w)
    q, k, v = f64(w.q), f64(w.k), f64(w.v)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)
    lse = torch.logsumexp((q @ k.transpose(-1, -2)) / math.sqrt(w.d), dim=-1).numpy()
    np.testing.assert_allclose(L, lse, rtol=0, atol=1e-12)


def test_oracle_full_causal_is_sdpa_causal():
    w = synth.random_case(8, B=1, Hq=4, Hkv=1, N=100, d=8, block=16, density=2.0, causal=True)
    O, _, _, _ = oracle_all(w)
    q, k, v = f64(w.q), f64(w.k).repeat_interleave(4, 1), f64(w.v).repeat_interleave(4, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def brute_force(w, perm_q, perm_k):
    """Pure-Python loops over tokens; InstaGen Eq. 2 (no max subtraction)."""
    Q = synth.bf16_bits_to_f32(w.q).astype(float)
    K = synth.bf16_bits_to_f32(w.k).astype(float)
    V = synth.bf16_bits_to_f32(w.v).astype(float)
    nb = w.nQB
    G = w.Hq // w.Hkv
    out = np.zeros((w.B, w.Hq, w.N, w.d))
    for b in range(w.B):
        for h in range(w.Hq):
            g = h // G
            bh, bg = b * w.Hq + h, b * w.Hkv + g
            posq = {int(perm_q[bh][i]): i for i in range(w.N)} if perm_q is not None else None
            posk = {int(perm_k[bg][i]): i for i in range(w.N)} if perm_k is not None else None
            for t in range(w.N):
                u = (posq[t] if posq else t) // w.block
                row = bh * nb + u
                num = [0.0] * w.d
                den = 0.0
                for s in range(w.N):
                    vb = (posk[s] if posk else s) // w.block
                    inmask = (w.mask[row][vb] != 0) if w.mask is not None else (w.T[row][vb] <= np.float32(w.p))
                    if not (inmask or vb == u):
                        continue
                    if w.causal and s > t:
                        continue
                    logit = sum(Q[b, h, t, c] * K[b, g, s, c] for c in range(w.d)) / math.sqrt(w.d)
                    if w.lw_map is not None:
                        logit += float(w.lw_map[row][vb])
                    e = math.exp(logit)
                    den += e
                    for c in range(w.d):
                        num[c] += e * V[b, g, s, c]
                for c in range(w.d):
                    out[b, h, t, c] = num[c] / den
    return out


@pytest.mark.parametrize("kw", [
    dict(B=1, Hq=2, Hkv=1, N=37, d=4, block=8, density=0.4, causal=True),
    dict(B=2, Hq=2, Hkv=2, N=45, d=6, block=8, density=0.3, permute=True, log_weights=True),
    dict(B=1, Hq=3, Hkv=3, N=48, d=8, block=4, density=0.2, use_T=True, log_weights=True),
])
def test_oracle_matches_brute_force(kw):
    w = synth.random_case(31, **kw)
    O, _, pq, pk = oracle_all(w)
    ref = brute_force(w, pq, pk)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_constant_values_give_constant_output():
    w = synth.random_case(9, B=1, Hq=2, Hkv=2, N=120, d=8, block=16, density=0.3, permute=True,
                          log_weights=True)
    w.v[:] = synth.f32_to_bf16_bits(np.array([1.75], dtype=np.float32))[0]
    O, _, _, _ = oracle_all(w)
    np.testing.assert_allclose(O, 1.75, rtol=0, atol=1e-12)


def test_zero_queries_give_weighted_block_mean():
    w = synth.random_case(10, B=1, Hq=1, Hkv=1, N=100, d=4, block=16, density=0.4, log_weights=True)
    w.q[:] = 0
    O, _, _, _ = oracle_all(w)
    nb = w.nQB
    V = synth.bf16_bits_to_f32(w.v[0, 0]).astype(float)
    for u in range(nb):
        keep = [vb for vb in range(nb) if w.mask[u][vb] or vb == u]
        wts = {vb: math.exp(float(w.lw_map[u][vb])) for vb in keep}
        sizes = {vb: min(w.block, w.N - vb * w.block) for vb in keep}
        num = sum(wts[vb] * V[vb * w.block: vb * w.block + sizes[vb]].sum(0) for vb in keep)
        den = sum(wts[vb] * sizes[vb] for vb in keep)
        for t in range(u * w.block, min(w.N, (u + 1) * w.block)):
            np.testing.assert_allclose(O[0, 0, t], num / den, rtol=0, atol=1e-12)


def test_log_weight_shift_moves_lse_only():
    w = synth.random_case(11, B=1, Hq=2, Hkv=2, N=96, d=8, block=16, density=0.5, log_weights=True)
    w.lw_map = (np.round(w.lw_map * 1024) / 1024).astype(np.float32)   # so that +-1 is exact in fp32
    rp, col, lw = oracle.build_csr(w.mask, None, 0, w.lw_map, w.nQB, True)
    O1, L1 = oracle.attn_full(w, rp, col, lw)
    lw2 = lw.copy()
    row = np.repeat(np.arange(len(rp) - 1), np.diff(rp))
    shift = (row % 3).astype(np.float32) - np.float32(1.0)   # -1, 0, +1 per row
    lw2 = (lw2 + shift).astype(np.float32)
    O2, L2 = oracle.attn_full(w, rp, col, lw2)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
    t = np.arange(w.B * w.Hq * w.N)
    r = (t // w.N) * w.nQB + (t % w.N) // w.block
    np.testing.assert_allclose(L2 - L1, (r % 3) - 1.0, rtol=0, atol=1e-12)


def test_log2_weight_equals_duplicated_block():
    """Weight 2 on block v (log-weight ln 2) is the same as listing a copy of
    block v's keys and values once more with weight 1."""
    blk, nb, d = 8, 6, 4
    w = synth.random_case(12, B=1, Hq=1, Hkv=1, N=blk * nb, d=d, block=blk, density=0.5)
    vdup = 2
    mask = w.mask.copy()
    mask[:, vdup] = 1
    lw_map = np.zeros(mask.shape, dtype=np.float32)
    lw_map[:, vdup] = np.float32(math.log(2.0))
    rp, col, lw = oracle.build_csr(mask, None, 0, lw_map, nb, True)
    O1, L1 = oracle.attn_full(w, rp, col, lw)
    # augmented problem: one extra key/value block that copies block vdup
    N2 = blk * (nb + 1)
    k2 = np.concatenate([w.k, w.k[:, :, vdup * blk:(vdup + 1) * blk]], axis=2)
    v2 = np.concatenate([w.v, w.v[:, :, vdup * blk:(vdup + 1) * blk]], axis=2)
    q2 = np.concatenate([w.q, np.zeros((1, 1, blk, d), np.uint16)], axis=2)
    mask2 = np.zeros((nb + 1, nb + 1), np.uint8)
    mask2[:nb, :nb] = mask
    mask2[:nb, nb] = 1
    rp2, col2, _ = oracle.build_csr(mask2, None, 0, None, nb + 1, True)
    rows = np.arange(w.N, dtype=np.int64)
    O2, L2 = oracle.attn_rows(q2, k2, v2, rp2, col2, None, blk, rows)
    # ln 2 is stored as float32: exp(fl(ln 2)) = 2 (1 + e) with |e| < 2^-24, so the
    # identity holds to that relative precision (|V| < 5 here), not to 1e-12.
    np.testing.assert_allclose(O1, O2, rtol=0, atol=5e-7)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-7)


def test_empty_row_gives_zero_and_minus_inf():
    w = synth.random_case(13, B=1, Hq=1, Hkv=1, N=64, d=4, block=16, density=0.0)
    rp, col, lw = oracle.build_csr(w.mask, None, 0, None, w.nQB, force_diag=False)
    assert rp[-1] == 0
    O, L = oracle.attn_rows(w.q, w.k, w.v, rp, np.zeros(1, np.int32), None, w.block,
                            np.arange(w.N, dtype=np.int64))
    assert np.all(O == 0) and np.all(np.isneginf(L))


def test_rows_sum_to_one():
    """With V = I-like one-hot columns the output row is the attention row
    restricted to those keys; summing over a full one-hot basis gives 1."""
    w = synth.random_case(14, B=1, Hq=1, Hkv=1, N=32, d=32, block=8, density=0.4, log_weights=True)
    w.v[:] = 0
    one = synth.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    w.v[0, 0, np.arange(32), np.arange(32)] = one      # V = identity -> O_t = softmax row t
    O, _, _, _ = oracle_all(w)
    np.testing.assert_allclose(O.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert np.all(O >= 0)
