"""A seeded random sweep of token-level attention over computational query
sets against the oracle, every listed query compared.

Each case draws from its own seed:

- batch, query and KV heads (GQA up to 4), and the sequence length;
- set size 64 or 128, the number of sets, and the query slots (some empty);
- a list length per set, from 0 to past the 2048-entry staging chunk, with out-of-range and duplicate entries;
- causal masking;
- head sharing: none, or runs of 2 or 4 query heads with identical sets.

Shared launches are also held to the bar against the per-head launch.  Bar
as for the other parity tests: max-abs 2e-2 / mean-abs 2e-3 on O, 1e-3 on
the LSE.
"""
import numpy as np
import pytest

from test_gpu_tok import _pair_identical_sets, _qkv, _run_and_compare

pytestmark = pytest.mark.gpu

N_CASES = 12


def draw(seed):
    g = np.random.default_rng(11000 + seed)
    Hkv = int(g.choice([1, 2]))
    G = int(g.choice([1, 2, 4]))
    Hq = Hkv * G
    B = int(g.choice([1, 1, 2]))
    N = int(g.integers(300, 5000))
    BQ = int(g.choice([64, 128]))
    causal = bool(g.random() < 0.4)
    share = 0
    if BQ == 64 and G % 2 == 0 and g.random() < 0.7:
        share = 4 if G % 4 == 0 and g.random() < 0.5 else 2
    C = int(g.integers(1, max(2, min(12, N // BQ))))
    lens = g.choice([0, 1, 7, 63, 64, 65, 129, 300, 700, 2049, 2100], size=C)
    return dict(seed=seed, B=B, Hq=Hq, Hkv=Hkv, N=N, BQ=BQ, C=C, causal=causal, share=share, lens=lens, g=g)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_sets_match_oracle(seed):
    c = draw(seed)
    desc = "B=%d Hq=%d Hkv=%d N=%d BQ=%d sets=%d causal=%d kv_share=%d lens=%s" % (
        c["B"], c["Hq"], c["Hkv"], c["N"], c["BQ"], c["C"], c["causal"], c["share"], list(c["lens"]))
    print("case tok sweep %d: %s" % (seed, desc), flush=True)
    q, k, v = _qkv(12000 + seed, c["B"], c["Hq"], c["Hkv"], c["N"])
    q_idx, kv_ptr, kv_idx = _pair_identical_sets(c["g"], c["B"], c["Hq"], c["N"], c["C"], c["BQ"], c["lens"],
                                                 run=max(c["share"], 1))
    _run_and_compare(q, k, v, q_idx, kv_ptr, kv_idx, c["causal"], "tok sweep %d" % seed,
                     kv_share=c["share"] if c["share"] else False)
