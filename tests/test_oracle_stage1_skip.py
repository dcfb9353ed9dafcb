"""Pins of the oracle's reading of WaveAlign's adaptive skip (section IV-E,
Runtime Coordination; section VI-F, Figure 13): stage 1 runs only when its
estimated latency reduction exceeds its overhead.  The fresh-block fraction
is checked against a brute-force set computation, the density against its
closed form, and the decision on both sides of every condition."""
import numpy as np
import pytest

import oracle

DEF = oracle.STAGE1_DEFAULTS


def csr_from_lists(lists):
    rp = np.zeros(len(lists) + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    col = np.concatenate([np.asarray(sorted(x), dtype=np.int32) for x in lists]) if rp[-1] else \
        np.zeros(0, np.int32)
    return rp, col


def random_lists(rng, BH, nQB, nKB, density, shared=False):
    lists = []
    for h in range(BH):
        base = rng.choice(nKB, size=max(1, int(round(density * nKB))), replace=False)
        for u in range(nQB):
            if shared:
                lists.append(base.tolist())
            else:
                lists.append(rng.choice(nKB, size=max(1, int(round(density * nKB))), replace=False).tolist())
    return lists


def brute_fresh(lists, BH, nQB):
    fresh = nnz = 0
    for h in range(BH):
        prev = set()
        for u in range(nQB):
            cur = set(lists[h * nQB + u])
            fresh += len(cur - prev)
            nnz += len(cur)
            prev = cur
    return fresh / nnz


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fresh_fraction_and_density_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    BH, nQB, nKB = 3, 17, 23
    lists = [rng.choice(nKB, size=int(rng.integers(0, nKB)), replace=False).tolist() for _ in range(BH * nQB)]
    rp, col = csr_from_lists(lists)
    _, st = oracle.stage1_decide(rp, col, BH, nQB, nKB, 17 * 128, 128, 128, 10, 256)
    assert st["fresh_fraction"] == pytest.approx(brute_fresh(lists, BH, nQB), abs=1e-15)
    assert st["density"] == pytest.approx(rp[-1] / (BH * nQB * nKB), abs=1e-15)


def test_every_listed_entry_counts():
    """An entry naming a block outside [0, nKB) is still a tile the attention
    kernels process: it counts in nnz, and it is fresh unless the previous row
    lists the same block."""
    rp, col = csr_from_lists([[0, 1], [1, 2]])
    col_bad = col.copy()
    col_bad[0] = 99
    _, a = oracle.stage1_decide(rp, col, 1, 2, 3, 256, 128, 128, 10, 256)
    _, b = oracle.stage1_decide(rp, col_bad, 1, 2, 3, 256, 128, 128, 10, 256)
    assert a["density"] == pytest.approx(4 / 6) and b["density"] == pytest.approx(4 / 6)
    assert a["fresh_fraction"] == pytest.approx(3 / 4)    # 0, 1 of row 0; 2 of row 1
    assert b["fresh_fraction"] == pytest.approx(3 / 4)    # 99, 1 of row 0; 2 of row 1


def big_case(shared, density=0.3, nQB=512, BH=64, seed=5):
    rng = np.random.default_rng(seed)
    lists = random_lists(rng, BH, nQB, nQB, density, shared=shared)
    return csr_from_lists(lists), BH, nQB


def test_reorders_long_dense_scattered_rows():
    """64 heads x 512 query blocks at 30 % density, every row its own random
    list (the order pairs almost nothing): 5.0M block pairs, ~41 ms of
    attention, so the estimated gain (~1.5 ms) exceeds stage 1's cost
    (~0.7 ms)."""
    (rp, col), BH, nQB = big_case(shared=False)
    run, st = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 256)
    assert st["fresh_fraction"] > 0.65 and st["gain_ms"] > st["cost_ms"]
    assert run


def test_skips_rows_that_already_share_their_blocks():
    (rp, col), BH, nQB = big_case(shared=True)
    run, st = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 256)
    assert st["fresh_fraction"] == pytest.approx(1.0 / nQB)   # only each head's first row is fresh
    assert not run


def test_skips_below_the_density_threshold():
    (rp, col), BH, nQB = big_case(shared=False, density=0.05)
    run, st = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 256)
    assert st["density"] < DEF[4] and not run
    # the same lists with the threshold lowered below their density
    run2, _ = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 256,
                                   params=DEF[:4] + (0.04,) + DEF[5:])
    assert run2 == (_["gain_ms"] > _["cost_ms"])


def test_skips_when_the_kv_of_a_head_fits_the_l2():
    (rp, col), BH, nQB = big_case(shared=False)
    # N = 8192 tokens at d = 128: K and V of a head take exactly 4 MiB
    run, st = oracle.stage1_decide(rp, col, BH, nQB, nQB, 8192, 128, 128, 10, 256)
    assert st["kv_bytes_per_head"] == 4 * 1024 * 1024 and not run
    run2, _ = oracle.stage1_decide(rp, col, BH, nQB, nQB, 8193, 128, 128, 10, 256)
    assert run2


def test_cost_and_gain_decide_at_the_margin():
    (rp, col), BH, nQB = big_case(shared=False)
    _, st = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 256)
    # more iterations make stage 1 dearer: past gain / cost times the default it is skipped
    k = int(np.ceil(10 * st["gain_ms"] / st["cost_ms"])) + 1
    run, st2 = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, k, 256)
    assert st2["cost_ms"] == pytest.approx(st["cost_ms"] * k / 10) and not run
    # a smaller expected gain per fresh visit does the same
    run3, st3 = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 256,
                                     params=(DEF[0] * st["cost_ms"] / st["gain_ms"] * 0.99,) + DEF[1:])
    assert st3["gain_ms"] < st3["cost_ms"] and not run3
    # more compute units shorten the attention and with it the gain
    _, st4 = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 512)
    assert st4["gain_ms"] == pytest.approx(st["gain_ms"] / 2)


def test_unsupported_shapes_are_skipped():
    rng = np.random.default_rng(3)
    nQB = 1100
    lists = [rng.choice(nQB, size=400, replace=False).tolist() for _ in range(8 * nQB)]
    rp, col = csr_from_lists(lists)
    cheap = DEF[:2] + (DEF[2] / 100, DEF[3] / 100) + DEF[4:]   # stage 1 made nearly free
    run, st = oracle.stage1_decide(rp, col, 8, nQB, nQB, nQB * 128, 128, 128, 10, 256, params=cheap)
    assert st["gain_ms"] > st["cost_ms"] and not run
    # the same statistics on a supported number of rows do reorder
    sub = [x for x in lists[:1024]]
    rp2, col2 = csr_from_lists([[v for v in x if v < 1024] for x in sub])
    run2, _ = oracle.stage1_decide(rp2, col2, 1, 1024, 1024, 1024 * 128, 128, 128, 10, 256, params=cheap)
    assert not run2   # 1024 x ceil(1024/32) words exceed the bitmask limit
    rp3, col3 = csr_from_lists([[v for v in x if v < 384] for x in lists[:384 * 8]])
    run3, st3 = oracle.stage1_decide(rp3, col3, 8, 384, 384, 384 * 128, 128, 128, 10, 256, params=cheap)
    assert run3 == (st3["gain_ms"] > st3["cost_ms"]) and run3


def test_block_and_head_dim_scale_the_attention_estimate():
    (rp, col), BH, nQB = big_case(shared=False, BH=4, nQB=64)
    _, a = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 128, 128, 128, 10, 256)
    _, b = oracle.stage1_decide(rp, col, BH, nQB, nQB, nQB * 64, 64, 64, 10, 256)
    assert b["t_attn_ms"] == pytest.approx(a["t_attn_ms"] / 8)
