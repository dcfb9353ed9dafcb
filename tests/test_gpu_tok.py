"""GPU parity of token-level attention over computational query sets (INTRA,
sections 3 and 4.8; MC-Sparse token-level KV selection), called through the
C ABI, against the oracle on the same seeded inputs.

Cases: random sets with lists of every awkward length (empty, 1, 63, 64,
65, over a 1024- and a 2048-entry staging chunk), out-of-range and duplicate
entries, empty query slots, GQA, full and causal masking, 64- and 128-query
sets; INTRA's Scatter, Gather 1 and Gather 0 maps; a token-selection workload
of MC-Sparse's shape.  The head-pair and head-quad launches (kv_share 2 or
4: the sets of each run of 2 or 4 consecutive query heads of a KV group are
identical, each gathered tile serves them all) are checked against the
oracle and, within the same bar, against the per-head launch.  Bar: max-abs 2e-2, mean-abs 2e-3 on O, 1e-3 on LSE; rows that no set
lists stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api
import synth
from parity_common import LSE_ABS, MAX_ABS, assert_within

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _qkv(seed, B, Hq, Hkv, N, d=128, scale_q=1.0):
    g = np.random.default_rng(seed)
    f = lambda H, s: synth.f32_to_bf16_bits((g.standard_normal((B, H, N, d)) * s).astype(np.float32))
    return f(Hq, scale_q), f(Hkv, 1.0), f(Hkv, 1.0)


def _run_and_compare(q, k, v, q_idx, kv_ptr, kv_idx, causal, label, slots=None, kv_share=False):
    B, Hq, N, d = q.shape
    C, BQ = q_idx.shape[1], q_idx.shape[2]
    args = (_gpu(q.view(np.int16)), _gpu(k.view(np.int16)), _gpu(v.view(np.int16)), _gpu(q_idx), _gpu(kv_ptr),
            _gpu(kv_idx))
    out, lse = api.attn_tok_fwd(*args, want_lse=True, causal=causal, kv_share=kv_share)
    torch.cuda.synchronize()
    if kv_share:
        # the per-head launch splits every tile's keys over two wavefronts and
        # merges them at the end; the shared launches walk whole tiles: same
        # values up to rounding order
        ref_out, ref_lse = api.attn_tok_fwd(*args, want_lse=True, causal=causal)
        torch.cuda.synchronize()
        a_ = synth.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16))
        b_ = synth.bf16_bits_to_f32(ref_out.cpu().numpy().view(np.uint16))
        assert np.abs(a_ - b_).max() <= MAX_ABS
        la, lb = lse.cpu().numpy(), ref_lse.cpu().numpy()
        assert np.array_equal(np.isnan(la), np.isnan(lb))
        fin = np.isfinite(la) & np.isfinite(lb)
        assert np.array_equal(np.isneginf(la), np.isneginf(lb))
        assert np.abs(la[fin] - lb[fin]).max(initial=0.0) <= LSE_ABS
    go = synth.bf16_bits_to_f32(out.cpu().numpy().view(np.uint16)).reshape(B * Hq, N, d)
    gl = lse.cpu().numpy()
    if slots is None:
        slots = np.arange(B * Hq * C * BQ, dtype=np.int64)
    ro, rl = oracle.attn_tok(q, k, v, q_idx, kv_ptr, kv_idx, slots, causal=causal)
    bh = slots // (C * BQ)
    t = q_idx.reshape(-1)[slots]
    ok = (t >= 0) & (t < N)
    got_o = go[bh[ok], t[ok]].astype(np.float64)
    err = np.abs(got_o - ro[ok])
    fin = np.isfinite(rl[ok])
    lerr = np.abs(gl[bh[ok], t[ok]][fin] - rl[ok][fin])
    assert np.all(np.isneginf(gl[bh[ok], t[ok]][~fin]))
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max=float(lerr.max() if lerr.size else 0),
                 rows=int(ok.sum()))
    _log("  %s: %s" % (label, stats))
    assert_within(stats)
    # rows of heads that no set lists keep their initial values
    listed = np.zeros((B * Hq, N), bool)
    qi = q_idx.reshape(B * Hq, -1)
    for h in range(B * Hq):
        v_ = qi[h][(qi[h] >= 0) & (qi[h] < N)]
        listed[h, v_] = True
    assert np.all(go[~listed] == 0) and np.all(np.isnan(gl[~listed]))


@pytest.mark.parametrize("BQ,causal,Hq,Hkv", [(64, False, 2, 2), (64, True, 4, 2), (128, False, 4, 1),
                                              (128, True, 2, 2)])
def test_random_sets(BQ, causal, Hq, Hkv):
    B, N = 1, 3000
    q, k, v = _qkv(BQ + causal + Hq, B, Hq, Hkv, N)
    g = np.random.default_rng(7 + BQ)
    C = 12
    q_idx = np.full((B * Hq, C, BQ), -1, np.int32)
    for h in range(B * Hq):
        pos = g.permutation(N)[:C * BQ - 9]                   # distinct positions, a few empty slots
        flat = np.full(C * BQ, -1, np.int32)
        flat[g.permutation(C * BQ)[:len(pos)]] = pos
        q_idx[h] = flat.reshape(C, BQ)
    lens = np.array([0, 1, 63, 64, 65, 200, 1100, 7, 128, 129, 500, 1024])
    lists = []
    for h in range(B * Hq):
        for c in range(C):
            keys = g.integers(0, N, size=lens[c]).astype(np.int32)
            if lens[c] > 10:
                keys[3] = -1                                  # outside the sequence
                keys[4] = N + 7
                keys[5] = keys[6]                             # a duplicate entry
            lists.append(keys)
    kv_ptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    kv_idx = np.concatenate(lists).astype(np.int32)
    _log("case tok random BQ=%d causal=%d Hq=%d Hkv=%d" % (BQ, causal, Hq, Hkv))
    _run_and_compare(q, k, v, q_idx, kv_ptr, kv_idx, causal, "random sets")


@pytest.mark.parametrize("causal", [False, True])
def test_intra_scatter(causal):
    B, Hq, Hkv, N = 1, 4, 2, 4096 + 40
    q, k, v = _qkv(21 + causal, B, Hq, Hkv, N)
    maps = synth.cqs_per_head(synth.cqs_scatter(N, 8, 64, causal), B * Hq)
    _log("case tok INTRA Scatter N=%d causal=%d" % (N, causal))
    _run_and_compare(q, k, v, *maps, causal, "scatter")


@pytest.mark.parametrize("causal", [False, True])
def test_intra_gather1(causal):
    B, Hq, Hkv, N = 1, 4, 2, 4096 + 40
    q, k, v = _qkv(23 + causal, B, Hq, Hkv, N)
    maps = synth.cqs_per_head(synth.cqs_gather1(N, 8, 64, causal), B * Hq)
    _log("case tok INTRA Gather 1 N=%d causal=%d" % (N, causal))
    _run_and_compare(q, k, v, *maps, causal, "gather1")


def _pair_identical_sets(g, B, Hq, N, C, BQ, lens, run=2):
    """Random sets drawn per run of `run` consecutive heads (its first head)
    and copied to the run's other heads."""
    q_idx = np.full((B * Hq, C, BQ), -1, np.int32)
    lists = [None] * (B * Hq * C)
    for h in range(0, B * Hq, run):
        pos = g.permutation(N)[:C * BQ - 5]
        flat = np.full(C * BQ, -1, np.int32)
        flat[g.permutation(C * BQ)[:len(pos)]] = pos
        for r in range(run):
            q_idx[h + r] = flat.reshape(C, BQ)
        for c in range(C):
            keys = g.integers(0, N, size=lens[c]).astype(np.int32)
            if lens[c] > 10:
                keys[3] = -1
                keys[4] = N + 7
                keys[5] = keys[6]
            for r in range(run):
                lists[(h + r) * C + c] = keys
    kv_ptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    return q_idx, kv_ptr, np.concatenate(lists).astype(np.int32)


@pytest.mark.parametrize("causal,Hq,Hkv", [(False, 2, 1), (True, 4, 2), (False, 8, 2)])
def test_head_pairs_random_sets(causal, Hq, Hkv):
    B, N, C, BQ = 1, 5000, 10, 64
    q, k, v = _qkv(60 + causal + Hq, B, Hq, Hkv, N)
    g = np.random.default_rng(61 + Hq)
    lens = np.array([0, 1, 63, 64, 65, 300, 2100, 7, 129, 2048])
    q_idx, kv_ptr, kv_idx = _pair_identical_sets(g, B, Hq, N, C, BQ, lens)
    _log("case tok head pairs random causal=%d Hq=%d Hkv=%d" % (causal, Hq, Hkv))
    _run_and_compare(q, k, v, q_idx, kv_ptr, kv_idx, causal, "head pairs", kv_share=True)


@pytest.mark.parametrize("causal,Hq,Hkv", [(False, 4, 1), (True, 8, 2)])
def test_head_quads_random_sets(causal, Hq, Hkv):
    B, N, C, BQ = 1, 5000, 10, 64
    q, k, v = _qkv(80 + causal + Hq, B, Hq, Hkv, N)
    g = np.random.default_rng(81 + Hq)
    lens = np.array([0, 1, 63, 64, 65, 300, 2100, 7, 129, 2048])
    q_idx, kv_ptr, kv_idx = _pair_identical_sets(g, B, Hq, N, C, BQ, lens, run=4)
    _log("case tok head quads random causal=%d Hq=%d Hkv=%d" % (causal, Hq, Hkv))
    _run_and_compare(q, k, v, q_idx, kv_ptr, kv_idx, causal, "head quads", kv_share=4)


@pytest.mark.parametrize("pattern", ["scatter", "gather1"])
def test_head_quads_intra(pattern):
    B, Hq, Hkv, N = 1, 8, 2, 4096 + 40
    q, k, v = _qkv(90 + len(pattern), B, Hq, Hkv, N)
    f = synth.cqs_scatter if pattern == "scatter" else synth.cqs_gather1
    maps = synth.cqs_per_head(f(N, 8, 64, True), B * Hq)
    _log("case tok head quads INTRA %s N=%d" % (pattern, N))
    _run_and_compare(q, k, v, *maps, True, pattern + " head quads", kv_share=4)


@pytest.mark.parametrize("pattern", ["scatter", "gather1"])
def test_head_pairs_intra(pattern):
    B, Hq, Hkv, N = 1, 8, 2, 4096 + 40
    q, k, v = _qkv(70 + len(pattern), B, Hq, Hkv, N)
    f = synth.cqs_scatter if pattern == "scatter" else synth.cqs_gather1
    maps = synth.cqs_per_head(f(N, 8, 64, True), B * Hq)
    _log("case tok head pairs INTRA %s N=%d" % (pattern, N))
    _run_and_compare(q, k, v, *maps, True, pattern + " head pairs", kv_share=True)


def test_intra_gather0():
    B, Hq, Hkv, H, W = 1, 2, 2, 64, 48
    N = H * W
    q, k, v = _qkv(31, B, Hq, Hkv, N, scale_q=2.0)
    maps = synth.cqs_per_head(synth.cqs_gather0(H, W), B * Hq)
    _log("case tok INTRA Gather 0 %dx%d" % (H, W))
    _run_and_compare(q, k, v, *maps, False, "gather0")


def test_token_selection():
    B, Hq, Hkv, N = 1, 2, 1, 8192
    q, k, v = _qkv(41, B, Hq, Hkv, N)
    maps = synth.cqs_per_head(synth.cqs_token_select(5, N, 128, 1500), B * Hq)
    C = maps[0].shape[1]
    rng = np.random.default_rng(3)
    slots = np.sort(rng.choice(B * Hq * C * 128, size=3000, replace=False)).astype(np.int64)
    _log("case tok token selection N=%d keys=1500" % N)
    _run_and_compare(q, k, v, *maps, False, "token selection", slots)


def test_extreme_scores():
    """Keys scaled by 1, 2 or 3 in runs of 256 tokens and every query +-8 times
    the same fixed key: scores near +-130, 260 and 390 (base 2).  Head 0's
    softmax puts its weight on the largest-scaled keys of each list; head 1's
    (negative queries) on the smallest-scaled ones, with every score far
    below zero.  Random lists of every awkward length, causal and not."""
    B, Hq, Hkv, N, BQ = 1, 2, 1, 3000, 64
    _, _, v = _qkv(71, B, Hq, Hkv, N)
    scale = 1.0 + (np.arange(N) // 256) % 3
    one = np.ones(128, np.float32)
    k = synth.f32_to_bf16_bits((scale[:, None] * one[None, :]).astype(np.float32)).reshape(B, Hkv, N, 128)
    q = np.empty((B, Hq, N, 128), np.uint16)
    q[0, 0] = synth.f32_to_bf16_bits(np.float32(8.0))
    q[0, 1] = synth.f32_to_bf16_bits(np.float32(-8.0))
    g = np.random.default_rng(72)
    C = 8
    q_idx = np.full((B * Hq, C, BQ), -1, np.int32)
    for h in range(B * Hq):
        q_idx[h] = g.permutation(N)[:C * BQ].reshape(C, BQ)
    lens = [1, 63, 64, 65, 300, 700, 129, 17]
    lists = [g.integers(0, N, size=lens[c]).astype(np.int32) for h in range(B * Hq) for c in range(C)]
    kv_ptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    kv_idx = np.concatenate(lists).astype(np.int32)
    for causal in (False, True):
        _log("case tok extreme scores causal=%d" % causal)
        _run_and_compare(q, k, v, q_idx, kv_ptr, kv_idx, causal, "extreme scores")
