"""WaveAlign's adaptive skip of stage 1 on the GPU (bsa_stage1_decide and the
gated bsa_spectral_order), against the oracle's reading of the rule: the
decision bit for bit, the statistics to the last bits; when the skip decides
for stage 1 the gated order equals the forced one, when it decides against it
the order is the identity and the schedule equals the one without stage 1; the
pipeline's "auto" mode equals the forced "on" or "off" mode it chose, bit for
bit."""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api, pipeline
import synth
from parity_common import run_gpu

pytestmark = pytest.mark.gpu

NAMES = ("fresh_fraction", "density", "t_attn_ms", "gain_ms", "cost_ms", "kv_bytes_per_head", "run")


def _log(msg):
    print(msg, flush=True)


def random_csr(rng, BH, nQB, density, shared):
    lists = []
    for h in range(BH):
        base = np.sort(rng.choice(nQB, size=max(1, int(density * nQB)), replace=False))
        for u in range(nQB):
            lists.append(base if shared else np.sort(rng.choice(nQB, size=max(1, int(density * nQB)),
                                                                 replace=False)))
    rp = np.zeros(BH * nQB + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(x) for x in lists])
    return rp, np.concatenate(lists).astype(np.int32)


def check(rp, col, BH, nQB, N, d, block, iters, params=None):
    cus = api.device_cus()
    prm = dict(zip(api.STAGE1_PARAM_NAMES, oracle.STAGE1_DEFAULTS))
    if params:
        prm.update(params)
    orun, ost = oracle.stage1_decide(rp, col, BH, nQB, nQB, N, d, block, iters, cus,
                                     params=tuple(prm[n] for n in api.STAGE1_PARAM_NAMES))
    rpd, cold = torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda()
    dec, st = api.stage1_decide(rpd, cold, BH, nQB, nQB, N, d, block, iters, params=params)
    st = st.cpu().numpy()
    assert int(dec.item()) == int(orun)
    for i, n in enumerate(NAMES):
        assert st[i] == pytest.approx(ost[n], rel=1e-13, abs=0.0), n
    return bool(orun), rpd, cold, dec


@pytest.mark.parametrize("shared,params,expect", [
    (False, None, True),                                   # long, dense, scattered rows: reorder
    (True, None, False),                                   # rows already share their blocks: skip
    (False, {"density_min": 0.5}, False),                  # below the density threshold: skip
    (False, {"gamma": 0.001}, False),                      # gain below cost: skip
])
def test_decision_and_gated_order(shared, params, expect):
    rng = np.random.default_rng(11)
    BH, nQB, block, d = 64, 512, 128, 128
    rp, col = random_csr(rng, BH, nQB, 0.3, shared)
    _log("case stage-1 decision shared=%s params=%s" % (shared, params))
    run, rpd, cold, dec = check(rp, col, BH, nQB, nQB * block, d, block, 10, params)
    assert run == expect
    gated, _ = api.spectral_order(rpd, cold, BH, nQB, nQB, 10, enable=dec)
    if run:
        forced, _ = api.spectral_order(rpd, cold, BH, nQB, nQB, 10)
        assert torch.equal(gated, forced)
    else:
        assert torch.equal(gated.cpu(), torch.arange(nQB, dtype=torch.int32).repeat(BH, 1))
        a = api.schedule(rpd, 1, BH, BH, nQB, 0, 8, row_perm=gated)
        b = api.schedule(rpd, 1, BH, BH, nQB, 0, 8)
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["tiny", "video_threshold", "llm_prefill", "clustered"])
def test_decision_on_the_workloads(name):
    w = synth.CONFIGS[name]()
    rp, col, _ = oracle.build_csr(w.mask, w.T, w.p, w.lw_map, w.nQB, w.force_diag)
    _log("case stage-1 decision on %s" % name)
    run, _, _, _ = check(rp, col, w.B * w.Hq, w.nQB, w.N, w.d, w.block, 10)
    assert not run   # measured on MI355X: stage 1 costs more than it saves on every workload here


@pytest.mark.parametrize("overlap", [False, True])
def test_auto_equals_the_mode_it_chose(overlap):
    w = synth.random_case(321, B=1, Hq=3, Hkv=3, N=1500, d=128, block=128, density=0.3, permute=True,
                          n_clusters=5)
    _log("case stage-1 auto vs forced, overlap=%s" % overlap)
    _, ra = run_gpu(w, schedule=True, n_xcd=8, stage1="auto", overlap=overlap)
    chosen = "on" if int(ra.stage1_decision.item()) else "off"
    _, rf = run_gpu(w, schedule=True, n_xcd=8, stage1=chosen, overlap=overlap)
    assert torch.equal(ra.order, rf.order)
    assert torch.equal(ra.out, rf.out)
    assert torch.equal(ra.lse, rf.lse)
    assert chosen == "off"   # 1500 tokens: K and V of a head fit one XCD's L2
