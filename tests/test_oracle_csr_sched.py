"""Pins of the oracle's integer routines: CSR builder, labels -> permutation,
row schedule, allowed-pair count.

* CSR: numpy's nonzero over the dense keep-matrix (library routine), the CRM
  bitmask forward iterator of ScalingAttention (section 7.3, Algorithm 2:
  clear-lowest-bit and count-trailing-zeros walk), the closed-form row sizes
  of the LLM prefill pattern, counting identities for T <= p.
* permutation: numpy's stable argsort (library routine).
* schedule: brute-force Python sort per bucket and structural invariants.
* pair count: the page-printed GFLOP figures of INTRA (golden fixture).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def keep_matrix(mask, T, p, nQB, force_diag=True):
    src = (mask != 0) if mask is not None else (T <= np.float32(p))
    keep = src.copy()
    if force_diag:
        r = np.arange(keep.shape[0])
        keep[r, r % nQB] = True
    return keep


@pytest.mark.parametrize("use_T", [False, True])
def test_csr_matches_numpy_nonzero(use_T):
    w = synth.random_case(21, B=2, Hq=3, Hkv=3, N=300, d=8, block=32, density=0.3, use_T=use_T,
                          log_weights=True)
    rp, col, lw = oracle.build_csr(w.mask, w.T, w.p, w.lw_map, w.nQB, True)
    keep = keep_matrix(w.mask, w.T, w.p, w.nQB)
    rr, cc = np.nonzero(keep)              # row-major, ascending columns
    np.testing.assert_array_equal(col, cc.astype(np.int32))
    np.testing.assert_array_equal(rp, np.concatenate([[0], np.cumsum(keep.sum(1))]).astype(np.int32))
    np.testing.assert_array_equal(lw.view(np.uint32), w.lw_map[rr, cc].view(np.uint32))


def test_csr_T_count_identity():
    w = synth.random_case(22, B=1, Hq=4, Hkv=4, N=512, d=8, block=32, density=0.2, use_T=True)
    rp, _, _ = oracle.build_csr(None, w.T, w.p, None, w.nQB, True)
    le = w.T <= np.float32(w.p)
    r = np.arange(w.R)
    diag_extra = int((~le[r, r % w.nQB]).sum())
    assert rp[-1] == int(le.sum()) + diag_extra


def test_csr_without_forced_diag_and_nan_threshold():
    T = np.array([[0.1, np.nan, 0.5], [np.nan, np.nan, np.nan], [0.5, 0.50001, -np.inf]], np.float32)
    rp, col, _ = oracle.build_csr(None, T, 0.5, None, 3, force_diag=False)
    assert rp.tolist() == [0, 2, 2, 4]
    assert col.tolist() == [0, 2, 0, 2]
    rp, col, _ = oracle.build_csr(None, T, 0.5, None, 3, force_diag=True)
    assert rp.tolist() == [0, 2, 3, 5] and col.tolist() == [0, 2, 1, 0, 2]


def test_lw_bits_copied_exactly():
    mask = np.ones((2, 4), np.uint8)
    lw_map = np.array([[-0.0, np.inf, 1e-42, -3.5], [np.float32(np.pi), -np.inf, 0.0, 7.0]], np.float32)
    rp, col, lw = oracle.build_csr(mask, None, 0, lw_map, 2, True)
    np.testing.assert_array_equal(lw.view(np.uint32), lw_map.reshape(-1).view(np.uint32))


def crm_walk(row_bits_words):
    """CRM forward iterator: words of 32 block flags; yield base + ctz, clearing
    the lowest set bit each step, advancing word by word."""
    out = []
    base = -32
    for w in row_bits_words:
        base += 32
        x = int(w)
        while x:
            low = x & -x
            out.append(base + low.bit_length() - 1)
            x &= x - 1
    return out


def test_csr_equals_crm_bitmask_walk():
    w = synth.random_case(23, B=1, Hq=2, Hkv=2, N=128 * 70, d=8, block=128, density=0.3)
    rp, col, _ = oracle.build_csr(w.mask, None, 0, None, w.nQB, True)
    keep = keep_matrix(w.mask, None, 0, w.nQB)
    nwords = -(-w.nQB // 32)
    for r in range(w.R):
        bits = np.zeros(nwords * 32, np.uint64)
        bits[:w.nQB] = keep[r]
        words = [int(sum(int(bits[i * 32 + j]) << j for j in range(32))) for i in range(nwords)]
        assert crm_walk(words) == col[rp[r]:rp[r + 1]].tolist()


def test_prefill_pattern_closed_form():
    nb, H = 512, 32
    pat = synth.prefill_pattern(nb)
    mask = np.broadcast_to(pat, (H, nb, nb)).reshape(-1, nb)
    rp, col, _ = oracle.build_csr(mask, None, 0, None, nb, True)
    sizes = np.diff(rp).reshape(H, nb)
    closed = np.array([min(u, 3) + 1 + u // 16 + (1 if (u > 3 and u % 16 != 0) else 0)
                       for u in range(nb)])
    assert np.all(sizes == closed[None])
    assert closed.sum() == 10455 and rp[-1] == 334560
    assert closed.min() == 1 and closed.max() == 36
    # block-lower-triangular: no listed block lies above the diagonal
    row = np.repeat(np.arange(H * nb), np.diff(rp)) % nb
    assert np.all(col <= row)


def test_tiny_has_64_blocks_per_head():
    w = synth.tiny()
    rp, _, _ = oracle.build_csr(w.mask, None, 0, None, w.nQB, True)
    per_head = np.diff(rp).reshape(w.Hq, w.nQB).sum(1)
    assert per_head.tolist() == [64, 64]


def test_perm_matches_stable_argsort():
    rng = np.random.default_rng(5)
    labels = rng.integers(-2, 9, size=(6, 1000), dtype=np.int32)   # includes out-of-range labels
    perm = oracle.perm_from_labels(labels, 7)
    key = np.where((labels >= 0) & (labels < 7), labels, 7)
    ref = np.argsort(key, axis=1, kind="stable").astype(np.int32)
    np.testing.assert_array_equal(perm, ref)
    # a permutation of 0..N-1 on every row
    assert np.all(np.sort(perm, 1) == np.arange(1000)[None])


def sched_brute(row_ptr, B, Hq, Hkv, nQB, W, n_xcd, row_perm=None, head_step=1):
    G = Hq // Hkv
    nnz = np.diff(row_ptr)
    logical = []
    blk = (lambda h, u: u) if row_perm is None else (lambda h, u: int(row_perm[h][u]))
    for b in range(B):
        for g in range(Hkv):
            seg = [(b * Hq + g * G + j) * nQB + blk(b * Hq + g * G + j, u) for u in range(nQB)
                   for j in range(0, G, head_step)]
            for s in range(0, len(seg), W):
                bucket = seg[s:s + W]
                logical += [r for _, _, r in sorted((-int(nnz[r]), i, r) for i, r in enumerate(bucket))]
    R = len(logical)
    if n_xcd <= 1:
        return np.array(logical, np.int32)
    counts = [len(range(x, R, n_xcd)) for x in range(n_xcd)]
    starts = np.concatenate([[0], np.cumsum(counts)])
    return np.array([logical[starts[i % n_xcd] + i // n_xcd] for i in range(R)], np.int32)


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", [(1, 4, 4, 37, 8, 1), (2, 8, 2, 20, 16, 8),
                                                   (1, 3, 1, 50, 7, 8), (1, 2, 2, 5, 100, 3)])
def test_schedule_matches_brute_force(B, Hq, Hkv, nQB, W, n_xcd):
    rng = np.random.default_rng(B * 100 + Hq + nQB)
    sizes = rng.integers(0, 9, size=B * Hq * nQB)
    row_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    order = oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, n_xcd)
    np.testing.assert_array_equal(order, sched_brute(row_ptr, B, Hq, Hkv, nQB, W, n_xcd))
    assert np.array_equal(np.sort(order), np.arange(B * Hq * nQB))


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", [(1, 4, 4, 37, 8, 1), (2, 8, 2, 20, 16, 8), (1, 3, 1, 50, 1, 1)])
def test_schedule_with_row_order_matches_brute_force(B, Hq, Hkv, nQB, W, n_xcd):
    rng = np.random.default_rng(B * 300 + Hq + nQB)
    sizes = rng.integers(0, 9, size=B * Hq * nQB)
    row_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    row_perm = np.stack([rng.permutation(nQB) for _ in range(B * Hq)]).astype(np.int32)
    order = oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, n_xcd, row_perm)
    np.testing.assert_array_equal(order, sched_brute(row_ptr, B, Hq, Hkv, nQB, W, n_xcd, row_perm))
    # identity order = no order; W = 1 keeps the given order untouched
    ident = np.tile(np.arange(nQB, dtype=np.int32), (B * Hq, 1))
    np.testing.assert_array_equal(oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, n_xcd, ident),
                                  oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, n_xcd))
    if W == 1 and n_xcd == 1 and Hq == Hkv:
        np.testing.assert_array_equal(order, (np.arange(B * Hq)[:, None] * nQB + row_perm).reshape(-1))


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", [(1, 4, 2, 37, 8, 1), (2, 8, 2, 20, 16, 8), (1, 32, 8, 64, 2048, 8)])
def test_schedule_of_head_pairs_matches_brute_force(B, Hq, Hkv, nQB, W, n_xcd):
    """Head step 2: only the first head of each pair sharing a KV head is
    scheduled (one launch per pair of identical rows)."""
    rng = np.random.default_rng(B * 700 + Hq + nQB)
    sizes = rng.integers(0, 9, size=B * Hq * nQB)
    row_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    order = oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, n_xcd, head_step=2)
    np.testing.assert_array_equal(order, sched_brute(row_ptr, B, Hq, Hkv, nQB, W, n_xcd, head_step=2))
    heads = order // nQB % Hq
    assert np.all(heads % 2 == 0) and len(set(order.tolist())) == B * Hq * nQB // 2
    with pytest.raises(ValueError):   # three query heads per KV head do not pair up
        oracle.schedule(row_ptr[:B * 3 * nQB + 1], B, 3, 1, nQB, W, n_xcd, head_step=2)


def _csr(lists):
    row_ptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    col = np.concatenate([np.asarray(x, np.int32) for x in lists]) if row_ptr[-1] else np.zeros(1, np.int32)
    return row_ptr, col


def _adaptive_brute(row_ptr, col, B, Hq, Hkv, nQB, n_xcd, head_step=1):
    """Per KV-group segment (nQB * G / head_step <= 2048 rows here): the
    sorted order or the sequence order, whichever has the smaller sum of
    |blocks of a row - blocks of the previous row| (exact sets: every block
    index below 256, so the signature is exact); the sequence order wins only
    when strictly smaller, and is then emitted sorted within 64-row windows
    (the fixed 64-row buckets)."""
    G = Hq // Hkv
    srt = sched_brute(row_ptr, B, Hq, Hkv, nQB, 2048, 1, head_step=head_step)
    seq = sched_brute(row_ptr, B, Hq, Hkv, nQB, 1, 1, head_step=head_step)
    win = sched_brute(row_ptr, B, Hq, Hkv, nQB, 64, 1, head_step=head_step)
    seg = nQB * G // head_step
    rows = [set(col[row_ptr[r]:row_ptr[r + 1]].tolist()) for r in range(len(row_ptr) - 1)]

    def cost(o):
        c, prev = 0, set()
        for r in o:
            c += len(rows[r] - prev)
            prev = rows[r]
        return c
    logical = []
    for s in range(0, len(srt), seg):
        a, b = srt[s:s + seg], seq[s:s + seg]
        logical += list(win[s:s + seg] if cost(b) < cost(a) else a)
    R = len(logical)
    if n_xcd <= 1:
        return np.array(logical, np.int32)
    counts = [len(range(x, R, n_xcd)) for x in range(n_xcd)]
    starts = np.concatenate([[0], np.cumsum(counts)])
    return np.array([logical[starts[i % n_xcd] + i // n_xcd] for i in range(R)], np.int32)


@pytest.mark.parametrize("B,Hq,Hkv,nQB,n_xcd,hs,kind", [
    (1, 4, 4, 37, 8, 1, "random"), (2, 8, 2, 40, 8, 1, "banded"), (1, 6, 3, 60, 3, 1, "clustered"),
    (1, 8, 2, 50, 8, 2, "banded"), (2, 4, 1, 33, 1, 2, "random"), (1, 2, 2, 70, 8, 1, "mixed")])
def test_adaptive_bucket_order_matches_set_differences(B, Hq, Hkv, nQB, n_xcd, hs, kind):
    """Schedule with W = 0 and the lists: each segment keeps the order whose
    consecutive rows share more blocks, against exact set differences."""
    rng = np.random.default_rng(nQB + 17 * Hq)
    lists = []
    for h in range(B * Hq):
        for u in range(nQB):
            if kind == "banded" or (kind == "mixed" and h % 2 == 0):
                lists.append(list(range(max(0, u - 2), min(nQB, u + 3))))
            elif kind == "clustered" or kind == "mixed":
                c = (u * 7) % 4   # cluster of the row, interleaved along the sequence
                lists.append(sorted(set((40 * c + np.arange(5 + 3 * c)).tolist())))
            else:
                lists.append(sorted(rng.choice(200, size=int(rng.integers(0, 12)), replace=False).tolist()))
    row_ptr, col = _csr(lists)
    got = oracle.schedule(row_ptr, B, Hq, Hkv, nQB, 0, n_xcd, head_step=hs, col=col)
    np.testing.assert_array_equal(got, _adaptive_brute(row_ptr, col, B, Hq, Hkv, nQB, n_xcd, hs))
    srt = oracle.schedule(row_ptr, B, Hq, Hkv, nQB, 2048, n_xcd, head_step=hs)
    seq = oracle.schedule(row_ptr, B, Hq, Hkv, nQB, 64, n_xcd, head_step=hs)
    if kind == "banded":        # neighbours share four of five blocks: the sequence order, in 64-row windows
        np.testing.assert_array_equal(got, seq)
    if kind == "clustered":     # equal-length rows of one cluster share every block: sorted
        np.testing.assert_array_equal(got, srt)
    # without the lists W = 0 is one sorted bucket per segment
    np.testing.assert_array_equal(oracle.schedule(row_ptr, B, Hq, Hkv, nQB, 0, n_xcd, head_step=hs), srt)


def test_schedule_buckets_longest_first():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, nQB, W = 1, 6, 6, 64, 10
    sizes = rng.integers(1, 40, size=B * Hq * nQB)
    row_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    order = oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, 1)
    for h in range(Hq):
        seg = order[h * nQB:(h + 1) * nQB]
        assert set(seg.tolist()) == set(range(h * nQB, (h + 1) * nQB))   # head-major
        for s in range(0, nQB, W):
            bk = seg[s:s + W]
            assert set(bk.tolist()) == set(range(h * nQB + s, h * nQB + min(nQB, s + W)))
            assert np.all(np.diff(sizes[bk]) <= 0)


def test_pair_count_matches_intra_printed_gflops():
    g = json.load(open(os.path.join(GOLDEN, "intra_flops.json")))
    for part in ("dense", "causal"):
        spec = g[part]
        for case in spec["cases"]:
            N, block = case["N"], 128
            nb = -(-N // block)
            rp, col, _ = oracle.build_csr(np.ones((nb, nb), np.uint8), None, 0, None, nb, True)
            pairs = oracle.count_pairs(rp, col, N, block, spec["causal"])
            gflop = 4 * spec["head_dim"] * pairs * spec["heads"] / 1e9
            assert math.floor(gflop * 10) / 10 == pytest.approx(case["gflop"], abs=1e-9), (part, case)


def test_pair_count_small_brute_force():
    w = synth.random_case(24, B=1, Hq=2, Hkv=2, N=70, d=4, block=16, density=0.5, causal=True)
    rp, col, _ = oracle.build_csr(w.mask, None, 0, None, w.nQB, True)
    got = oracle.count_pairs(rp, col, w.N, w.block, True)
    keep = keep_matrix(w.mask, None, 0, w.nQB)
    ref = 0
    for r in range(w.R):
        u = r % w.nQB
        for t in range(u * 16, min(w.N, u * 16 + 16)):
            for s in range(w.N):
                if keep[r, s // 16] and s <= t:
                    ref += 1
    assert got == ref
