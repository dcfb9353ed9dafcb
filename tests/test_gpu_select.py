"""GPU parity of MC-Sparse's exact token-level KV selection ("The MC-Sparse
Architecture" and Algorithm 1: a dense pass gives each query's log-sum-exp,
the selection sums every key's attention probability over a query group and
keeps the K keys of largest mass), called through the C ABI, against the
oracle on the same seeded inputs.

* top-K: bit-exact against the oracle's sort on the same float32 rows
  (planted ties, signed zeros, denormals, k = 1 .. k > n, every row length
  class of the kernel up to the 75,600-key rows of Wan2.1-14B at 720p).
* group mass: the GPU takes its log-sum-exp from the library's own dense
  attention pass, the oracle computes its own in fp64.  Each mass is a sum of
  positive terms exp(x - l); an error e in l (the attention parity bar allows
  1e-3) scales each term by exp(e), so the bar is a relative 2e-3 plus 1e-6
  absolute for fp32 rounding of tiny sums.
* end to end: the GPU's top-K of its own mass equals the oracle's top-K of
  that same mass bit for bit, and differs from the oracle's top-K of the fp64
  mass only by keys whose fp64 mass lies within the mass bar of the K-th
  largest (near-ties).
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api
import synth

pytestmark = pytest.mark.gpu

RTOL, ATOL = 2e-3, 1e-6


def _log(msg):
    print(msg, flush=True)


def _gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _rows(seed, rows, n):
    g = np.random.default_rng(seed)
    x = g.random((rows, n)).astype(np.float32)
    if rows > 1:
        x[1] = 0.5                                           # all equal
    if rows > 2:
        x[2] = np.round(x[2] * 3) / 3                        # few distinct values
    if rows > 3:
        x[3] = g.standard_normal(n).astype(np.float32)
        x[3, ::7] = -0.0
        x[3, ::11] = 0.0                                     # signed zeros tie
    if rows > 4:
        x[4] = (g.random(n) * 1e-40).astype(np.float32)      # denormals
    return x


@pytest.mark.parametrize("n", [1, 300, 4096, 4097, 20000, 32768, 32769, 75600])
def test_topk_rows_bit_exact(n):
    x = _rows(n, 5, n)
    xd = _gpu(x)
    for k in sorted({1, 7, max(1, n // 7), n // 2 + 1, n, n + 3}):
        _log("topk n=%d k=%d" % (n, k))
        got = api.topk_rows(xd, k)
        torch.cuda.synchronize()
        ref = oracle.topk(x, k)
        np.testing.assert_array_equal(got.cpu().numpy(), ref)


def test_topk_rows_strided_and_empty():
    x = _rows(5, 4, 1000)
    big = np.zeros((4, 1040), np.float32)
    big[:, :1000] = x
    xd = _gpu(big)[:, :1000]                                 # row stride 1040
    np.testing.assert_array_equal(api.topk_rows(xd, 33).cpu().numpy(), oracle.topk(x, 33))
    assert api.topk_rows(xd, 0).shape == (4, 0)


def _groups(seed, BH, N, BQ, empty=5):
    """Each head's positions in a seeded random order, cut into sets of BQ
    (query groups of arbitrary positions, as a clustering leaves them), with
    a few empty slots and a ragged last set."""
    g = np.random.default_rng(seed)
    C = -(-(N + empty) // BQ)
    q_idx = np.full((BH, C, BQ), -1, np.int32)
    for h in range(BH):
        flat = np.full(C * BQ, -1, np.int32)
        slots = g.permutation(C * BQ)[:N]
        flat[np.sort(slots)] = g.permutation(N)
        q_idx[h] = flat.reshape(C, BQ)
    return q_idx


def _dense_lse(qd, kd, vd, causal):
    B, Hq, N, d = qd.shape
    nQB = -(-N // 128)
    mask = torch.ones((B * Hq, nQB, nQB), dtype=torch.uint8, device="cuda")
    if causal:
        mask = torch.tril(mask)
    row_ptr, col, _ = api.build_csr(mask=mask.reshape(B * Hq * nQB, nQB), nQB=nQB)
    out, lse = api.attn_fwd(qd, kd, vd, row_ptr, col, 128, want_lse=True, causal=causal)
    return out, lse


def _qkv(seed, B, Hq, Hkv, N, d=128, scale_q=1.0):
    g = np.random.default_rng(seed)
    f = lambda H, s: synth.f32_to_bf16_bits((g.standard_normal((B, H, N, d)) * s).astype(np.float32))
    return f(Hq, scale_q), f(Hkv, 1.0), f(Hkv, 1.0)


def _check_mass(got, ref, label):
    err = np.abs(got.astype(np.float64) - ref)
    bound = RTOL * ref + ATOL
    _log("  %s: max_abs %.3g, max rel %.3g, rows %d" % (label, err.max(), (err / np.maximum(ref, 1e-30)).max(),
                                                        got.shape[0]))
    bad = err > bound
    assert not bad.any(), "%d entries outside the bar, worst %s" % (bad.sum(), np.unravel_index(
        np.argmax(err - bound), err.shape))


@pytest.mark.parametrize("BQ,causal,B,Hq,Hkv,scale_q", [(128, False, 1, 4, 2, 1.0), (128, True, 1, 2, 2, 1.0),
                                                        (64, False, 2, 2, 1, 3.0), (64, True, 1, 4, 1, 3.0)])
def test_group_mass_matches_oracle(BQ, causal, B, Hq, Hkv, scale_q):
    N = 1000                                                 # ragged against 128-key tiles
    q, k, v = _qkv(BQ + 10 * causal + Hq, B, Hq, Hkv, N, scale_q=scale_q)
    q_idx = _groups(3 + BQ, B * Hq, N, BQ)
    _log("group_mass BQ=%d causal=%d B=%d Hq=%d Hkv=%d" % (BQ, causal, B, Hq, Hkv))
    qd, kd, vd = (_gpu(a.view(np.int16)) for a in (q, k, v))
    _, lse = _dense_lse(qd, kd, vd, causal)
    qi = _gpu(q_idx)
    got = api.group_mass(qd, kd, lse, qi, causal=causal)
    part = api.group_mass(qd, kd, lse, qi, keys=(130, 777), causal=causal)
    torch.cuda.synchronize()
    ref = oracle.group_mass(q, k, q_idx, causal=causal)
    _check_mass(got.cpu().numpy(), ref, "all keys")
    np.testing.assert_array_equal(part.cpu().numpy(), got.cpu().numpy()[:, 130:777])


def _near_tie_check(sel, ref_sel, ref_mass, K):
    """sel and ref_sel differ only by keys whose fp64 mass is within the bar
    of the K-th largest fp64 mass."""
    for r in range(sel.shape[0]):
        a, b = set(sel[r].tolist()), set(ref_sel[r].tolist())
        if a == b:
            continue
        kth = np.sort(ref_mass[r])[::-1][K - 1]
        diff = np.array(sorted(a ^ b))
        band = 2 * (RTOL * kth + ATOL)
        assert np.all(np.abs(ref_mass[r, diff] - kth) <= band), (r, diff[:8], ref_mass[r, diff[:8]], kth)


@pytest.mark.parametrize("BQ", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_selection_end_to_end(causal, BQ):
    B, Hq, Hkv, N, K = 1, 2, 1, 2000, 300                   # few groups: the key range is split
    q, k, v = _qkv(40 + causal, B, Hq, Hkv, N, scale_q=2.0)
    q_idx = _groups(41 + BQ, B * Hq, N, BQ)
    qd, kd, vd = (_gpu(a.view(np.int16)) for a in (q, k, v))
    _, lse = _dense_lse(qd, kd, vd, causal)
    mass = api.group_mass(qd, kd, lse, _gpu(q_idx), causal=causal)
    sel = api.topk_rows(mass, K)
    torch.cuda.synchronize()
    gm, gs = mass.cpu().numpy(), sel.cpu().numpy()
    np.testing.assert_array_equal(gs, oracle.topk(gm, K))    # same fp32 input: bit-exact
    ref = oracle.group_mass(q, k, q_idx, causal=causal)
    _check_mass(gm, ref, "mass")
    _near_tie_check(gs, oracle.topk(ref, K), ref, K)
    assert np.all(np.diff(gs, axis=1) > 0)


def test_wan14b_720p_sampled():
    """MC-Sparse's kernel workload shape (Wan2.1-14B at 720p: 40 heads, 75,600
    tokens, d = 128, groups of 128, K at 15 % density), the launches the
    benchmark times; sampled groups checked against the oracle."""
    B, Hq, Hkv, N, BQ = 1, 40, 40, 75600, 128
    K = int(0.15 * N)
    q, k, v = _qkv(75, B, Hq, Hkv, N)
    q_idx = _groups(76, B * Hq, N, BQ, empty=0)
    qd, kd, vd = (_gpu(a.view(np.int16)) for a in (q, k, v))
    _log("wan14b: dense pass")
    _, lse = _dense_lse(qd, kd, vd, False)
    _log("wan14b: mass")
    mass = api.group_mass(qd, kd, lse, _gpu(q_idx))
    _log("wan14b: top-K")
    sel = api.topk_rows(mass, K)
    torch.cuda.synchronize()
    C = q_idx.shape[1]
    picks = [(0, 0), (17, 301), (39, C - 1)]                 # (head, group), the last one ragged
    rows = [h * C + c for h, c in picks]
    gm = mass[rows].cpu().numpy()
    gs = sel[rows].cpu().numpy()
    np.testing.assert_array_equal(gs, oracle.topk(gm, K))
    for (h, c), r in zip(picks, range(len(rows))):
        _log("  oracle head %d group %d" % (h, c))
        ref = oracle.group_mass(q[:, h:h + 1], k[:, h:h + 1], q_idx[h:h + 1, c:c + 1])
        _check_mass(gm[r:r + 1], ref, "head %d group %d" % (h, c))
        _near_tie_check(gs[r:r + 1], oracle.topk(ref, K), ref, K)


def test_llama3_8b_32k_causal_sampled():
    """Causal selection with GQA at the LLaMA-3.1-8B prefill shape (32 query
    heads over 8 KV heads, 32,768 tokens, groups of 128 consecutive tokens,
    K = 4096): every launch at full size, sampled groups against the oracle.
    The first group has mass on its first 128 keys only, so most of its
    selection is the lowest-indexed zero-mass keys."""
    B, Hq, Hkv, N, BQ, K = 1, 32, 8, 32768, 128, 4096
    q, k, v = _qkv(32, B, Hq, Hkv, N)
    C = N // BQ
    q_idx = np.broadcast_to(np.arange(N, dtype=np.int32).reshape(1, C, BQ), (B * Hq, C, BQ)).copy()
    qd, kd, vd = (_gpu(a.view(np.int16)) for a in (q, k, v))
    _log("llama 32k: dense causal pass")
    _, lse = _dense_lse(qd, kd, vd, True)
    _log("llama 32k: mass + top-K")
    mass = api.group_mass(qd, kd, lse, _gpu(q_idx), causal=True)
    sel = api.topk_rows(mass, K)
    torch.cuda.synchronize()
    picks = [(0, 0), (13, 100), (31, C - 1)]
    rows = [h * C + c for h, c in picks]
    gm = mass[rows].cpu().numpy()
    gs = sel[rows].cpu().numpy()
    np.testing.assert_array_equal(gs, oracle.topk(gm, K))
    for r, (h, c) in enumerate(picks):
        g = h // (Hq // Hkv)
        _log("  oracle head %d (kv %d) group %d" % (h, g, c))
        ref = oracle.group_mass(q[:, h:h + 1], k[:, g:g + 1], q_idx[h:h + 1, c:c + 1], causal=True)
        assert np.all(gm[r, (c + 1) * BQ:] == 0) and np.all(ref[0, (c + 1) * BQ:] == 0)
        _check_mass(gm[r:r + 1], ref, "head %d group %d" % (h, c))
        _near_tie_check(gs[r:r + 1], oracle.topk(ref, K), ref, K)


def test_dead_queries_add_nothing():
    """A query whose log-sum-exp is -inf or NaN adds nothing: the masses equal,
    bit for bit, those of the same sets with that query's slot emptied (the
    summation order is fixed)."""
    B, Hq, Hkv, N, BQ = 1, 2, 2, 700, 128
    q, k, v = _qkv(91, B, Hq, Hkv, N)
    q_idx = _groups(92, B * Hq, N, BQ)
    qd, kd, vd = (_gpu(a.view(np.int16)) for a in (q, k, v))
    _, lse = _dense_lse(qd, kd, vd, False)
    dead = q_idx.copy()
    lse_dead = lse.clone()
    g = np.random.default_rng(93)
    for h in range(B * Hq):
        pos = g.choice(N, size=40, replace=False)
        lse_dead[h, pos[:20]] = float("-inf")
        lse_dead[h, pos[20:]] = float("nan")
        dead[h][np.isin(dead[h], pos)] = -1
    for causal in (False, True):
        a = api.group_mass(qd, kd, lse_dead, _gpu(q_idx), causal=causal)
        b = api.group_mass(qd, kd, lse, _gpu(dead), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a, b), causal
