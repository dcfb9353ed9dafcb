"""GPU parity at small sizes: every step of the HIP path, called through the C
ABI, against the CPU oracle on the same seeded inputs, element by element.

Integer outputs (CSR, permutations, schedule) must match bit for bit;
attention outputs within max-abs 2e-2 / mean-abs 2e-3 (bf16 inputs, fp32
accumulation, probabilities and outputs rounded to bf16), LSE within 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api, pipeline
import synth
from parity_common import (assert_within, bf16_tensor_to_f32, compare_rows, oracle_csr, oracle_perms, sample_rows,
                           run_gpu)

pytestmark = pytest.mark.gpu

CASES = {
    "b128_d128_tail_lw": dict(B=1, Hq=2, Hkv=2, N=1000, d=128, block=128, density=0.4, log_weights=True),
    "b64_d64_gqa_T": dict(B=2, Hq=4, Hkv=2, N=700, d=64, block=64, density=0.3, use_T=True),
    "b128_d128_causal_gqa": dict(B=1, Hq=4, Hkv=1, N=900, d=128, block=128, density=0.6, causal=True),
    "b128_d128_perm_lw": dict(B=1, Hq=3, Hkv=3, N=1200, d=128, block=128, density=0.3, permute=True,
                              log_weights=True, n_clusters=7),
    "b64_d128_perm_gqa": dict(B=1, Hq=2, Hkv=1, N=777, d=128, block=64, density=0.35, permute=True),
    "b128_d64_full": dict(B=1, Hq=2, Hkv=2, N=640, d=64, block=128, density=2.0),
    "b128_d128_peaky": dict(B=1, Hq=2, Hkv=2, N=1100, d=128, block=128, density=0.5, q_scale=3.0,
                            log_weights=True),
    "single_partial_block": dict(B=1, Hq=2, Hkv=1, N=50, d=128, block=64, density=1.0, causal=True),
}


def make(name, seed=500):
    return synth.random_case(seed + list(CASES).index(name), **CASES[name])


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_csr_bit_exact(name):
    w = make(name)
    _log("case %s: csr" % name)
    dw = pipeline.to_device(w)
    rp, col, lw = api.build_csr(dw.mask, dw.T, dw.p, dw.lw_map, dw.nQB, True, want_lw=True)
    orp, ocol, olw = oracle.build_csr(w.mask, w.T, w.p, w.lw_map, w.nQB, True, want_lw=True)
    np.testing.assert_array_equal(rp.cpu().numpy(), orp)
    np.testing.assert_array_equal(col.cpu().numpy(), ocol)
    np.testing.assert_array_equal(lw.cpu().numpy().view(np.uint32), olw.view(np.uint32))


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("sched,fuse,vdm", [(True, True, True), (False, False, True), (True, True, False),
                                            (False, False, False)])
def test_attention_matches_oracle(name, sched, fuse, vdm):
    w = make(name)
    _log("case %s: attention sched=%s fuse=%s v_dim_major=%s" % (name, sched, fuse, vdm))
    _, res = run_gpu(w, schedule=sched, fuse_scatter=fuse, fuse_gather=fuse, n_xcd=8, wave_rows=16, v_dim_major=vdm)
    pq, pk = oracle_perms(w)
    rows = np.arange(w.B * w.Hq * w.N, dtype=np.int64)
    stats = compare_rows(w, res, rows, pq, pk)
    _log("  %s" % stats)
    assert_within(stats)


def test_tiny_config_full():
    w = synth.tiny()
    _log("case tiny: attention")
    _, res = run_gpu(w, schedule=True, n_xcd=8)
    rows = np.arange(w.B * w.Hq * w.N, dtype=np.int64)
    stats = compare_rows(w, res, rows)
    _log("  %s" % stats)
    assert_within(stats)


@pytest.mark.parametrize("vdm", [True, False])
def test_order_invariance_and_determinism(vdm):
    w = make("b128_d128_perm_lw")
    _log("case determinism v_dim_major=%s" % vdm)
    # one row per launch entry: every row is computed the same way whatever
    # the launch order, so the outputs are bit-identical
    _, r1 = run_gpu(w, schedule=False, fuse_scatter=True, v_dim_major=vdm)
    _, r2 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=5, fuse_scatter=True, v_dim_major=vdm, pair_rows=False)
    _, r3 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=5, fuse_scatter=False, v_dim_major=vdm,
                    pair_rows=False)
    _, r4 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=5, fuse_scatter=False, fuse_gather=False,
                    v_dim_major=vdm, pair_rows=False)
    a = r1.out.cpu().numpy()
    assert np.array_equal(a, r2.out.cpu().numpy())
    assert np.array_equal(a, r3.out.cpu().numpy())
    assert np.array_equal(a, r4.out.cpu().numpy())       # fused query gather == explicit gather
    assert np.array_equal(r1.lse.cpu().numpy(), r3.lse.cpu().numpy())
    assert np.array_equal(r1.lse.cpu().numpy(), r4.lse.cpu().numpy())
    # paired launch entries (the default schedule): the same tables give the
    # same bits, fused or explicit scatter
    _, p1 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=5, fuse_scatter=True, v_dim_major=vdm)
    _, p2 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=5, fuse_scatter=False, v_dim_major=vdm)
    assert (p1.order2 is not None) == vdm
    assert torch.equal(p1.out, p2.out) and torch.equal(p1.lse, p2.lse)


@pytest.mark.parametrize("name", ["b128_d128_perm_lw", "b64_d64_gqa_T", "b128_d128_causal_gqa"])
def test_overlapped_step_is_bit_identical(name):
    """The two-stream step (CSR without a host round trip) gives the same bits
    as the one-stream step."""
    w = make(name)
    _log("case overlapped step %s" % name)
    _, r1 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0)
    _, r2 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0, overlap=True)
    nnz = int(r1.row_ptr[-1].item())
    assert torch.equal(r1.row_ptr, r2.row_ptr) and torch.equal(r1.col, r2.col[:nnz])
    assert torch.equal(r1.order, r2.order)
    assert (r1.order2 is None) == (r2.order2 is None)
    if r1.order2 is not None:
        assert torch.equal(r1.order2, r2.order2)
    assert torch.equal(r1.out, r2.out) and torch.equal(r1.lse, r2.lse)


@pytest.mark.parametrize("BH,N,C", [(3, 75600, 64), (2, 5000, 1023), (2, 5000, 1024), (1, 9000, 3000),
                                    (4, 17, 5), (2, 64 * 16 * 8 + 1, 7)])
def test_perm_from_labels_bit_exact(BH, N, C):
    """Both kernel shapes (16 wavefronts up to 1023 clusters, 4 above), out-of-range
    labels, segments shorter than one load batch and exactly one batch long."""
    rng = np.random.default_rng(N + C)
    labels = rng.integers(-2, C + 2, size=(BH, N), dtype=np.int32)
    _log("case perm BH=%d N=%d C=%d" % (BH, N, C))
    got = api.perm_from_labels(torch.from_numpy(labels).cuda(), C).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.perm_from_labels(labels, C))


def test_perm_and_row_gather_bit_exact():
    rng = np.random.default_rng(77)
    labels = rng.integers(-1, 40, size=(6, 3001), dtype=np.int32)   # includes out-of-range
    _log("case perm")
    got = api.perm_from_labels(torch.from_numpy(labels).cuda(), 37).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.perm_from_labels(labels, 37))
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, 3, 3001, 128), dtype=np.float32))
    xt = torch.from_numpy(x.view(np.int16)).cuda()
    perm = torch.from_numpy(got).cuda()
    y = api.permute_rows(xt, perm)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint16),
                                  np.take_along_axis(x, got.reshape(2, 3, 3001)[..., None], 2))
    z = api.unpermute_rows(y, perm)
    np.testing.assert_array_equal(z.cpu().numpy(), xt.cpu().numpy())
    # gather + transpose into the dim-major layout, zero columns past N
    for pp in (perm, None):
        vt = api.transpose_rows(xt, pp, ld=3072).cpu().numpy().view(np.uint16)
        g = np.take_along_axis(x, got.reshape(2, 3, 3001)[..., None], 2) if pp is not None else x
        np.testing.assert_array_equal(vt[..., :3001], np.swapaxes(g, 2, 3))
        assert np.all(vt[..., 3001:] == 0)


@pytest.mark.parametrize("B,Hq,Hkv,nQB,W,n_xcd", [(1, 4, 4, 37, 8, 1), (2, 8, 2, 20, 16, 8),
                                                   (1, 3, 1, 50, 7, 8), (1, 40, 40, 591, 32, 8),
                                                   (1, 32, 8, 512, 2048, 8)])
def test_schedule_bit_exact(B, Hq, Hkv, nQB, W, n_xcd):
    rng = np.random.default_rng(B * 1000 + Hq + nQB)
    sizes = rng.integers(0, 40, size=B * Hq * nQB)
    row_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    _log("case schedule %s" % ((B, Hq, Hkv, nQB, W, n_xcd),))
    got = api.schedule(torch.from_numpy(row_ptr).cuda(), B, Hq, Hkv, nQB, W, n_xcd).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, n_xcd))


@pytest.mark.parametrize("kind,B,Hq,Hkv,nQB,n_xcd,hs,perm", [
    ("random", 1, 4, 4, 37, 8, 1, False), ("banded", 2, 8, 2, 300, 8, 1, False),
    ("clustered", 1, 6, 3, 591, 8, 1, False), ("banded", 1, 8, 2, 512, 8, 2, False),
    ("mixed", 1, 4, 4, 700, 3, 1, True), ("random", 1, 2, 1, 1500, 8, 1, False)])
def test_adaptive_schedule_bit_exact(kind, B, Hq, Hkv, nQB, n_xcd, hs, perm):
    """wave_rows = 0 with the block lists: per segment the sorted or the
    sequence order by the block signatures of consecutive rows (block indices
    beyond 256 alias in the signature; both sides take the same bits)."""
    rng = np.random.default_rng(nQB + Hq)
    lists = []
    for h in range(B * Hq):
        for u in range(nQB):
            if kind == "banded" or (kind == "mixed" and h % 2 == 0):
                lists.append(list(range(max(0, u - 3), min(nQB, u + 4))))
            elif kind in ("clustered", "mixed"):
                c = (u * 7) % 5
                lists.append(sorted(set(((97 * c + 3 * np.arange(6 + 4 * c)) % nQB).tolist())))
            else:
                lists.append(sorted(rng.choice(nQB, size=int(rng.integers(0, 30)), replace=False).tolist()))
    row_ptr = np.concatenate([[0], np.cumsum([len(x) for x in lists])]).astype(np.int32)
    col = np.concatenate([np.asarray(x, np.int32) for x in lists])
    row_perm = np.stack([rng.permutation(nQB) for _ in range(B * Hq)]).astype(np.int32) if perm else None
    _log("case adaptive schedule %s" % ((kind, B, Hq, Hkv, nQB, n_xcd, hs, perm),))
    got = api.schedule(torch.from_numpy(row_ptr).cuda(), B, Hq, Hkv, nQB, 0, n_xcd, head_step=hs,
                       col=torch.from_numpy(col).cuda(),
                       row_perm=None if row_perm is None else torch.from_numpy(row_perm).cuda()).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.schedule(row_ptr, B, Hq, Hkv, nQB, 0, n_xcd, row_perm, hs, col))


def test_empty_rows_write_zero_and_minus_inf():
    w = synth.random_case(9, B=1, Hq=2, Hkv=2, N=300, d=128, block=128, density=0.0)
    w.force_diag = False
    w.mask[1] = 1
    _log("case empty rows")
    _, res = run_gpu(w, schedule=False)
    out = bf16_tensor_to_f32(res.out).reshape(2, 300, 128)
    lse = res.lse.cpu().numpy().reshape(2, 300)
    assert np.all(out[0, :128] == 0) and np.all(np.isneginf(lse[0, :128]))
    rows = np.arange(600, dtype=np.int64)
    assert_within(compare_rows(w, res, rows))


def test_zero_queries_and_constant_values():
    w = synth.random_case(10, B=1, Hq=2, Hkv=2, N=520, d=128, block=128, density=0.4, log_weights=True)
    w.q[:] = 0
    _log("case Q=0")
    _, res = run_gpu(w, schedule=False)
    assert_within(compare_rows(w, res, np.arange(2 * 520, dtype=np.int64)))
    w.v[:] = synth.f32_to_bf16_bits(np.array([0.625], np.float32))[0]
    _, res = run_gpu(w, schedule=True, n_xcd=8)
    # P is rounded to bf16 for the PV product while the row sum uses fp32 P, so
    # a constant V comes back within one bf16 ulp (2^-8 at 0.625), not exactly
    assert np.abs(bf16_tensor_to_f32(res.out) - np.float32(0.625)).max() <= 2.0 ** -8


@pytest.mark.parametrize("block,causal,vdm", [(128, True, True), (128, False, True), (64, True, True),
                                            (128, True, False)])
def test_underflowing_scores_with_an_empty_key_half(block, causal, vdm):
    """Every score at about -130 in base-2 units (all keys equal, every query
    -8 times that key), each row listing only its diagonal block.  Under the
    causal mask the first half of each query block has no allowed key in the
    upper half of the tile, and the partial last block (50 tokens) has none
    without it: a key range with nothing accumulated must not take part in
    the merge, whatever running max it holds.  The softmax is uniform over the
    allowed keys, so O is their mean of V."""
    w = synth.random_case(77 + block + causal, B=1, Hq=2, Hkv=2, N=2 * 128 + 50, d=128, block=block,
                          density=0.0, causal=causal)
    w.k[:] = synth.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    w.q[:] = synth.f32_to_bf16_bits(np.array([-8.0], np.float32))[0]
    _log("case underflowing scores block=%d causal=%d v_dim_major=%d" % (block, causal, vdm))
    _, res = run_gpu(w, schedule=False, v_dim_major=vdm)
    stats = compare_rows(w, res, np.arange(2 * w.N, dtype=np.int64))
    _log("  %s" % stats)
    assert_within(stats)


@pytest.mark.parametrize("block,vdm", [(128, True), (64, True), (128, False)])
def test_scores_far_above_the_running_max(block, vdm):
    """Every row lists every block; the keys of block v are (v mod 3 + 1)
    times a fixed key and every query is 8 times that key, so a row's scores
    sit near 130, 260 and 390 (base 2) by block.  The first exponentials
    overflow, later blocks raise the running max by far more than the
    exponent range after something has been accumulated, and the rescale
    factor of the earlier blocks underflows to zero.  The softmax then puts
    all its weight on the keys of the top blocks, whose scores are equal."""
    N = 5 * block + 23
    w = synth.random_case(91 + block, B=1, Hq=2, Hkv=1, N=N, d=128, block=block, density=2.0)
    k0 = synth.f32_to_bf16_bits(np.array([1.0, 2.0, 3.0], np.float32))
    for v in range(-(-N // block)):
        w.k[:, :, v * block:(v + 1) * block] = k0[v % 3]
    w.q[:] = synth.f32_to_bf16_bits(np.array([8.0], np.float32))[0]
    _log("case scores far above the running max block=%d v_dim_major=%d" % (block, vdm))
    _, res = run_gpu(w, schedule=True, n_xcd=8, v_dim_major=vdm)
    stats = compare_rows(w, res, np.arange(2 * w.N, dtype=np.int64))
    _log("  %s" % stats)
    assert_within(stats)


@pytest.mark.parametrize("block,d,nblocks", [(128, 128, 1100), (64, 64, 1100)])
def test_long_rows_span_list_chunks(block, d, nblocks):
    """Rows of over a thousand KV blocks: the kernels stage a row's CSR list in
    LDS in chunks, so these rows cross chunk boundaries (online-softmax state
    carried across chunks).  Sampled rows: one random query block per head and
    the tail block."""
    w = synth.random_case(600 + block, B=1, Hq=2, Hkv=1, N=block * nblocks - 37, d=d, block=block, density=0.97,
                          log_weights=True)
    _log("case long rows block=%d d=%d N=%d" % (block, d, w.N))
    _, res = run_gpu(w, schedule=True, n_xcd=8, wave_rows=0)
    rp = res.row_ptr.cpu().numpy()
    assert np.diff(rp).max() > 1024
    rows = sample_rows(w, seed=3, per_block=False)
    stats = compare_rows(w, res, rows)
    _log("  %s" % stats)
    assert_within(stats)


def _check_spectral(gperm, gang, operm, oang):
    """Orders equal except among rows whose angles tie within 1e-9 (fp64 sums
    in different orders on the two sides); angles equal within 1e-9."""
    d = np.abs(((gang - oang) + np.pi) % (2 * np.pi) - np.pi)
    assert d.max() < 1e-9, d.max()
    for h in range(gperm.shape[0]):
        if np.array_equal(gperm[h], operm[h]):
            continue
        bad = np.nonzero(gperm[h] != operm[h])[0]
        a = oang[h][operm[h][bad]]
        b = oang[h][gperm[h][bad]]
        assert np.abs(a - b).max() < 1e-9, (h, bad[:8])
        assert sorted(gperm[h].tolist()) == list(range(gperm.shape[1]))


@pytest.mark.parametrize("BH,nQB,density,iters", [(3, 100, 0.2, 10), (2, 591, 0.15, 10), (4, 37, 0.5, 15),
                                                  (1, 600, 0.05, 6)])
def test_spectral_order_matches_oracle(BH, nQB, density, iters):
    rng = np.random.default_rng(BH * 1000 + nQB)
    protos = rng.random((5, nQB)) < density
    lab = rng.integers(0, 5, size=BH * nQB)
    m = (protos[lab] ^ (rng.random((BH * nQB, nQB)) < 0.03)).astype(np.uint8)
    rows, cols = np.nonzero(m)
    rp = np.concatenate([[0], np.cumsum(m.sum(1))]).astype(np.int32)
    col = cols.astype(np.int32)
    _log("case spectral BH=%d nQB=%d" % (BH, nQB))
    gp, ga = api.spectral_order(torch.from_numpy(rp).cuda(), torch.from_numpy(col).cuda(), BH, nQB, nQB, iters,
                                want_angle=True)
    operm, oang = oracle.spectral_order(rp, col, BH, nQB, nQB, iters)
    _check_spectral(gp.cpu().numpy(), ga.cpu().numpy(), operm, oang)


def test_schedule_with_row_order_bit_exact():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, nQB, W, n_xcd = 2, 8, 2, 40, 16, 8
    sizes = rng.integers(0, 30, size=B * Hq * nQB)
    row_ptr = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    row_perm = np.stack([rng.permutation(nQB) for _ in range(B * Hq)]).astype(np.int32)
    _log("case schedule with row order")
    got = api.schedule(torch.from_numpy(row_ptr).cuda(), B, Hq, Hkv, nQB, W, n_xcd,
                       row_perm=torch.from_numpy(row_perm).cuda()).cpu().numpy()
    np.testing.assert_array_equal(got, oracle.schedule(row_ptr, B, Hq, Hkv, nQB, W, n_xcd, row_perm))


def test_stage1_schedule_leaves_outputs_unchanged():
    w = make("b128_d128_perm_lw")
    _log("case stage-1 schedule invariance")
    _, r1 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=16, stage1="off", pair_rows=False)
    _, r2 = run_gpu(w, schedule=True, n_xcd=8, wave_rows=16, stage1="on", stage1_iters=8, pair_rows=False)
    assert not np.array_equal(r1.order.cpu().numpy(), r2.order.cpu().numpy())
    assert np.array_equal(r1.out.cpu().numpy(), r2.out.cpu().numpy())
    assert np.array_equal(r1.lse.cpu().numpy(), r2.lse.cpu().numpy())


@pytest.mark.parametrize("block,d,vdm", [(128, 128, True), (128, 64, True), (64, 128, True), (128, 128, False),
                                         (64, 64, False)])
def test_minus_inf_log_weights(block, d, vdm):
    """Log-weights of -inf remove a listed block from the softmax (its
    exponentials are 0).  Blocks with lw = -inf are scattered over the rows,
    and one row has -inf on every listed block, the diagonal included: its
    queries have no allowed key, so O = 0 and LSE = -inf there."""
    N = 3 * block + 37
    w = synth.random_case(4242 + block + d + vdm, B=1, Hq=2, Hkv=1, N=N, d=d, block=block, density=0.6,
                          log_weights=True)
    rng = np.random.default_rng(7)
    drop = rng.random(w.lw_map.shape) < 0.3
    w.lw_map[drop] = -np.inf
    full = w.nQB + 1                      # head 1, query block 1
    w.lw_map[full, :] = -np.inf
    _log("case -inf log-weights block=%d d=%d v_dim_major=%d" % (block, d, vdm))
    _, res = run_gpu(w, schedule=True, n_xcd=8, v_dim_major=vdm)
    rows = np.arange(w.B * w.Hq * N, dtype=np.int64)
    stats = compare_rows(w, res, rows)
    _log("  %s" % stats)
    assert_within(stats)
    out = bf16_tensor_to_f32(res.out).reshape(w.Hq, N, d)
    lse = res.lse.cpu().numpy().reshape(w.Hq, N)
    assert np.all(out[1, block:2 * block] == 0)
    assert np.all(np.isneginf(lse[1, block:2 * block]))
