"""Index data from the device that points outside its range is guarded in the
attention kernels: a corrupt entry reads nothing and writes nothing, and the
rest of the output is unaffected.

One launch per kernel shape carries every kind of corruption at once:

- CSR block indices at or past nKB, or negative: the entry takes no part,
  as if it were not listed (the oracle runs on the remaining entries);
- launch-table entries outside [0, R): that slot computes nothing, so the
  row it replaced is never written;
- gather-permutation entries outside [0, N): that position's query row reads
  as zeros (the oracle runs with that query set to zero);
- scatter-permutation entries outside [0, N): that position's output and
  LSE are not written.

Unwritten outputs keep a sentinel bit pattern, bit for bit.  Written ones
are held to the usual bar against the oracle: max-abs 2e-2, mean-abs 2e-3
on O and 1e-3 on the LSE.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_mask_amd import api, pipeline
import synth
from parity_common import assert_within, compare_rows, oracle_perms

pytestmark = pytest.mark.gpu

O_SENTINEL = 0x4123          # bf16 bits of 10.1875
LSE_SENTINEL = 12345.0


@pytest.mark.parametrize("block,d,vdm,share", [(128, 128, True, False), (128, 64, True, False),
                                               (64, 128, True, False), (128, 128, False, False),
                                               (128, 128, True, True)])
def test_corrupt_device_indices_touch_nothing(block, d, vdm, share):
    Hq, Hkv, N = 2, 1, 6 * block + 37
    w = synth.random_case(5150 + block + d + 2 * vdm + 4 * share, B=1, Hq=Hq, Hkv=Hkv, N=N, d=d, block=block,
                          density=0.5, permute=True, log_weights=True, n_clusters=5)
    nQB = w.nQB
    R = Hq * nQB
    if share:   # the pair kernel serves heads 0 and 1 from head 0's rows: make them identical
        w.mask[nQB:] = w.mask[:nQB]
        w.lw_map[nQB:] = w.lw_map[:nQB]
    print("case corrupt indices block=%d d=%d v_dim_major=%d kv_share=%d" % (block, d, vdm, share), flush=True)
    pq, pk = oracle_perms(w)
    dw = pipeline.to_device(w)
    pq_d = torch.from_numpy(pq.reshape(-1)).cuda()
    pk_d = torch.from_numpy(pk.reshape(-1)).cuda()
    kp = api.permute_rows(dw.k, pk_d)
    v = api.transpose_rows(dw.v, pk_d, ld=nQB * block) if vdm else api.permute_rows(dw.v, pk_d)
    rp, col, lw = api.build_csr(dw.mask, None, 0.0, dw.lw_map, nQB, True, want_lw=True)
    order = api.schedule(rp, 1, Hq, Hkv, nQB, 0, 8, col=col, head_step=2 if share else 1)
    rp_h, col_h, lw_h = rp.cpu().numpy(), col.cpu().numpy(), lw.cpu().numpy()
    rng = np.random.default_rng(block + d + vdm + share)

    # block indices: about a fifth of the entries, alternately past nKB and negative
    # (with head pairs the same entries of both heads' rows, which the kernel reads once)
    bad = np.zeros(col_h.size, bool)
    rows_drawn = range(nQB) if share else range(R)
    for r in rows_drawn:
        e0, e1 = rp_h[r], rp_h[r + 1]
        pick = rng.random(e1 - e0) < 0.2
        bad[e0:e1] |= pick
        if share:
            bad[rp_h[r + nQB]:rp_h[r + nQB + 1]] |= pick
    col_bad = col_h.copy()
    idx = np.flatnonzero(bad)
    col_bad[idx] = np.where(np.arange(idx.size) % 2 == 0, nQB + 3, -2)
    keep = ~bad
    rp_ok = np.concatenate([[0], np.cumsum([keep[rp_h[r]:rp_h[r + 1]].sum() for r in range(R)])]).astype(np.int32)
    csr_ok = (rp_ok, col_h[keep].astype(np.int32), lw_h[keep].astype(np.float32))

    # launch table: a quarter of the slots replaced by entries outside [0, R)
    order_h = order.cpu().numpy().copy()
    slots = rng.choice(order_h.size, size=max(1, order_h.size // 4), replace=False)
    skipped = order_h[slots].copy()
    order_h[slots] = np.array([-1, R + 5, 1 << 30], np.int32)[np.arange(slots.size) % 3]
    skipped_rows = set(int(r) for r in skipped)
    if share:
        skipped_rows |= set(int(r) + nQB for r in skipped)

    # gather and scatter entries outside [0, N) at a few positions per head
    gq, sq = pq.copy(), pq.copy()
    g_pos = [rng.choice(N, size=4, replace=False) for _ in range(Hq)]
    s_pos = [rng.choice(N, size=4, replace=False) for _ in range(Hq)]
    for h in range(Hq):
        gq[h, g_pos[h]] = np.array([-1, N, N + 2, -7], np.int32)
        sq[h, s_pos[h]] = np.array([-3, N + 9, N, -1], np.int32)

    out = torch.empty_like(dw.q)
    out.view(torch.int16).fill_(O_SENTINEL)
    lse = torch.full((Hq, N), LSE_SENTINEL, dtype=torch.float32, device="cuda")
    api.attn_fwd(dw.q, kp, v, rp, torch.from_numpy(col_bad).cuda(), block, lw=lw,
                 order=torch.from_numpy(order_h).cuda(), scatter_perm_q=torch.from_numpy(sq.reshape(-1)).cuda(),
                 gather_perm_q=torch.from_numpy(gq.reshape(-1)).cuda(), out=out, lse=lse, v_dim_major=vdm,
                 kv_share=share)
    torch.cuda.synchronize()

    # which original tokens get written: position i of head h, if its row was
    # launched and its scatter entry is valid, writes token pq[h][i]
    written = np.zeros((Hq, N), bool)
    for h in range(Hq):
        for i in range(N):
            if (h * nQB + i // block) in skipped_rows or not (0 <= sq[h, i] < N):
                continue
            written[h, pq[h, i]] = True
    o_bits = out.view(torch.int16).cpu().numpy().view(np.uint16).reshape(Hq, N, d)
    l_h = lse.cpu().numpy()
    assert np.all(o_bits[~written] == O_SENTINEL), "an unwritten output row was written"
    assert np.all(l_h[~written] == np.float32(LSE_SENTINEL)), "an unwritten LSE was written"
    assert written.sum() < Hq * N and written.sum() > Hq * N // 2

    # the oracle on the remaining entries, with the corrupt gathers' queries set to zero
    wz = synth.Workload(w.name, w.B, Hq, Hkv, N, d, block, w.q.copy(), w.k, w.v, causal=False)
    for h in range(Hq):
        wz.q[0, h, pq[h, g_pos[h]]] = 0
    rows = np.flatnonzero(written.reshape(-1)).astype(np.int64)

    class Res:
        pass
    res = Res()
    res.out, res.lse = out, lse
    stats = compare_rows(wz, res, rows, pq, pk, csr_ok)
    print("  %s, %d entries corrupt, %d rows written" % (stats, int(bad.sum()), int(written.sum())), flush=True)
    assert_within(stats)
