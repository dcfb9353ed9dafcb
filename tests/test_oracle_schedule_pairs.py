"""Pins of the oracle's paired launch tables (oracle.schedule_pairs).

The pairing is checked against a different formulation of the same rule:
maximal runs of consecutive query blocks of a head whose rows are identical
(found with numpy row comparisons) pair up from the run's start, (u0, u0+1),
(u0+2, u0+3), ...; a run of odd length leaves its last row alone.  Around it:
every row is served exactly once, paired rows list identical blocks and
log-weights, entries are longest-first by tile count (within windows of 64
positions when the position order is kept), the empty entries close each
bucket, the tables equal oracle.schedule's once pairs are split, and a
hand-worked six-row head.
"""
import numpy as np
import pytest

import oracle
import synth


def lists(rp, col):
    return [tuple(col[rp[r]:rp[r + 1]].tolist()) for r in range(len(rp) - 1)]


def runs_pairs(rp, col, lw, B, Hq, Hkv, nQB, W):
    """Pairs (r, r') by the run formulation, buckets of W positions of the
    KV-group segment (head inner)."""
    G = Hq // Hkv
    W = W or 2048
    L = lists(rp, col)
    LW = None if lw is None else [lw[rp[r]:rp[r + 1]].view(np.uint32).tobytes() for r in range(len(rp) - 1)]
    ident = lambda a, c: L[a] == L[c] and (LW is None or LW[a] == LW[c])
    pairs = set()
    for b in range(B):
        for g in range(Hkv):
            seg = [(b * Hq + g * G + j) * nQB + u for u in range(nQB) for j in range(G)]
            for k0 in range(0, len(seg), W):
                bucket = seg[k0:k0 + W]
                for j in range(G):
                    chain = bucket[j::G]          # one head's rows, consecutive query blocks
                    i = 0
                    while i < len(chain):
                        e = i
                        while e + 1 < len(chain) and ident(chain[e], chain[e + 1]):
                            e += 1
                        for a in range(i, e, 2):  # the run chain[i..e] pairs from its start
                            if a + 1 <= e:
                                pairs.add((chain[a], chain[a + 1]))
                        i = e + 1
    return pairs


def block_case(seed, B, Hq, Hkv, nQB, n_patterns, lw=False):
    """Rows drawn from a few block patterns, in runs, so that identical
    consecutive rows are common."""
    g = np.random.default_rng(seed)
    pats = [np.sort(g.choice(nQB, size=int(g.integers(1, nQB + 1)), replace=False)) for _ in range(n_patterns)]
    rows = []
    R = B * Hq * nQB
    while len(rows) < R:
        p = pats[int(g.integers(0, n_patterns))]
        rows += [p] * int(g.integers(1, 6))
    rows = rows[:R]
    rp = np.zeros(R + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in rows])
    col = np.concatenate(rows).astype(np.int32)
    w = None
    if lw:
        w = np.where(g.random(col.size) < 0.05, np.float32(-0.5), np.float32(0.0)).astype(np.float32)
    return rp, col, w


CASES = [(1, 1, 1, 40, 0, 1), (2, 3, 3, 37, 0, 8), (1, 4, 2, 33, 0, 4), (1, 2, 2, 150, 64, 8),
         (2, 4, 1, 50, 0, 1), (1, 1, 1, 300, 0, 8)]


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", CASES)
@pytest.mark.parametrize("with_lw", [False, True])
def test_pairs_equal_run_formulation(B, Hq, Hkv, nQB, W, n_xcd, with_lw):
    rp, col, lw = block_case(nQB * 7 + Hq, B, Hq, Hkv, nQB, 4, with_lw)
    o1, o2 = oracle.schedule_pairs(rp, col, B, Hq, Hkv, nQB, W, n_xcd, lw=lw)
    got = {(int(a), int(c)) for a, c in zip(o1, o2) if c >= 0}
    assert got == runs_pairs(rp, col, lw, B, Hq, Hkv, nQB, W)
    served = np.concatenate([o1[o1 >= 0], o2[o2 >= 0]])
    assert np.array_equal(np.sort(served), np.arange(B * Hq * nQB))
    L = lists(rp, col)
    for a, c in got:
        assert L[a] == L[c]
        if lw is not None:
            assert np.array_equal(lw[rp[a]:rp[a + 1]].view(np.uint32), lw[rp[c]:rp[c + 1]].view(np.uint32))
        assert c == a + 1                      # next query block of the same head
    assert np.all((o1 >= 0) | (o2 < 0))       # an empty entry has no second row


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W", [(1, 1, 1, 40, 0), (2, 3, 3, 37, 0), (1, 4, 2, 33, 16),
                                            (1, 2, 2, 150, 64)])
def test_bucket_structure(B, Hq, Hkv, nQB, W):
    """Without the XCD deal the table is the buckets one after another: the
    entries longest-first by tile count (or, when the position order was
    kept, longest-first within windows of 64 positions), then as many empty
    entries as the bucket has pairs."""
    rp, col, _ = block_case(5 + nQB, B, Hq, Hkv, nQB, 3)
    o1, o2 = oracle.schedule_pairs(rp, col, B, Hq, Hkv, nQB, W, 1)
    ln = np.diff(rp)
    G = Hq // Hkv
    seg = G * nQB
    Wb = W or 2048
    for s0 in range(0, B * Hq * nQB, seg):
        for b0 in range(s0, s0 + seg, Wb):
            n = min(Wb, s0 + seg - b0)
            a, c = o1[b0:b0 + n], o2[b0:b0 + n]
            m = int((a >= 0).sum())
            assert np.all(a[:m] >= 0) and np.all(a[m:] < 0) and np.all(c[m:] < 0)
            assert n - m == int((c >= 0).sum())
            cost = np.where(c[:m] >= 0, 2, 1) * ln[a[:m]]
            if W:
                assert np.all(np.diff(cost) <= 0)
            else:
                # sorted, or position order sorted within 64-position windows:
                # the position of an entry is that of its first row in the segment
                pos = np.array([(int(r) // nQB - (s0 // nQB)) % G + G * (int(r) % nQB) for r in a[:m]])
                win = (pos - (b0 - s0)) // 64
                if not np.all(np.diff(cost) <= 0):
                    assert np.all(np.diff(win) >= 0)
                    for w_ in np.unique(win):
                        assert np.all(np.diff(cost[win == w_]) <= 0)


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", [(1, 1, 1, 40, 16, 1), (2, 3, 3, 37, 64, 8)])
def test_no_identical_rows_equals_plain_schedule(B, Hq, Hkv, nQB, W, n_xcd):
    """With no two consecutive rows identical there is nothing to pair: the
    tables are oracle.schedule's order and -1 everywhere."""
    R = B * Hq * nQB
    # row (.., u) lists blocks u .. u + k: consecutive query blocks start at
    # different blocks, lengths vary
    rows = [np.arange(r % nQB, min(nQB, r % nQB + 1 + (7 * r) % 5), dtype=np.int32) for r in range(R)]
    rp = np.zeros(R + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in rows])
    col = np.concatenate(rows).astype(np.int32)
    o1, o2 = oracle.schedule_pairs(rp, col, B, Hq, Hkv, nQB, W, n_xcd)
    assert np.all(o2 == -1)
    assert np.array_equal(o1, oracle.schedule(rp, B, Hq, Hkv, nQB, W, n_xcd))


def test_hand_worked_head():
    """One head of six query blocks: lists [0,1] [0,1] [0,1] [2] [2,3,4]
    [2,3,4].  Blocks 0 and 1 pair (cost 4), block 2 is alone (2), block 3
    alone (1), blocks 4 and 5 pair (6): entries (4,5) (0,1) (2) (3), then two
    empty entries."""
    rows = [[0, 1], [0, 1], [0, 1], [2], [2, 3, 4], [2, 3, 4]]
    rp = np.array([0] + list(np.cumsum([len(x) for x in rows])), dtype=np.int32)
    col = np.array(sum(rows, []), dtype=np.int32)
    for W in (0, 8):
        o1, o2 = oracle.schedule_pairs(rp, col, 1, 1, 1, 6, W, 1)
        assert o1.tolist() == [4, 0, 2, 3, -1, -1]
        assert o2.tolist() == [5, 1, -1, -1, -1, -1]
    # a different log-weight on one entry of block 0 breaks the (0, 1) pair:
    # (1, 2) pairs instead (cost 4), block 0 is alone (2)
    lw = np.zeros(col.size, dtype=np.float32)
    lw[1] = -1.0
    o1, o2 = oracle.schedule_pairs(rp, col, 1, 1, 1, 6, 8, 1, lw=lw)
    assert o1.tolist() == [4, 1, 0, 3, -1, -1]
    assert o2.tolist() == [5, 2, -1, -1, -1, -1]


def test_clustered_workload_pairs_most_rows():
    """On the clustered workload's lists most rows sit in runs of identical
    rows (query blocks inside one cluster): the tables serve every row once
    and pair more than 80 % of them."""
    w = synth.clustered(H=4, N=16384, C=16)
    rp, col, _ = oracle.build_csr(None, w.T, w.p, None, w.nQB, True)
    o1, o2 = oracle.schedule_pairs(rp, col, 1, 4, 4, w.nQB, 0, 8)
    served = np.concatenate([o1[o1 >= 0], o2[o2 >= 0]])
    assert np.array_equal(np.sort(served), np.arange(4 * w.nQB))
    assert 2 * int((o2 >= 0).sum()) > 0.8 * 4 * w.nQB
