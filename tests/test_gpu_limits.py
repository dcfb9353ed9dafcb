"""GPU parity at the largest sizes the kernels accept: one head of N = 4,194,100
tokens, d = 128, so that Q, K and the dim-major V each span just under the
2^30 bytes that 32-bit buffer offsets address, with a ragged last block.

Each 128-query block row lists two KV blocks: its own and a far one, so that
K and V tiles are read from the top of the address range.  Checked on
sampled rows against the oracle: the CSR-fed kernel, the same lists as CRM
rows, and a token-level set whose queries and keys sit at the ends of the
sequence.  Inputs are seeded N(0, 1) draws made on the device and copied to
the host for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_mask_amd import api
import synth
from parity_common import assert_within

pytestmark = pytest.mark.gpu

N = 4_194_100
D = 128
BLOCK = 128


def _log(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def big():
    g = torch.Generator(device="cuda").manual_seed(99)
    q, k, v = (torch.randn((1, 1, N, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
               for _ in range(3))
    host = tuple(x.cpu().view(torch.int16).numpy().view(np.uint16) for x in (q, k, v))
    nqb = -(-N // BLOCK)
    far = (np.arange(nqb, dtype=np.int64) * 7919 + nqb // 2) % nqb
    cols = []
    for u in range(nqb):
        cols.append(sorted({u, int(far[u])}))
    row_ptr = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    col = np.concatenate(cols).astype(np.int32)
    yield q, k, v, host, row_ptr, col, nqb
    del q, k, v
    torch.cuda.empty_cache()


def _rows(nqb):
    rng = np.random.default_rng(5)
    blocks = np.unique(np.concatenate([[0, 1, nqb - 2, nqb - 1], rng.integers(0, nqb, size=12)]))
    rows = []
    for u in blocks:
        t0 = u * BLOCK
        rows += [t0, min(N - 1, t0 + 77), min(N - 1, t0 + BLOCK - 1)]
    return np.unique(np.array(rows, dtype=np.int64))


def _compare(out, lse, host, row_ptr, col, rows, label):
    qh, kh, vh = host
    ro, rl = oracle.attn_rows(qh, kh, vh, row_ptr, col, None, BLOCK, rows)
    go = synth.bf16_bits_to_f32(out.reshape(-1, D)[torch.from_numpy(rows).cuda()].cpu().view(torch.int16)
                                .numpy().view(np.uint16)).astype(np.float64)
    gl = lse.reshape(-1)[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    err = np.abs(go - ro)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max=float(np.abs(gl - rl).max()),
                 rows=len(rows))
    _log("  %s: %s" % (label, stats))
    assert_within(stats)


def test_csr_and_crm_at_the_address_limit(big):
    q, k, v, host, row_ptr, col, nqb = big
    _log("case limits N=%d (CSR, CRM)" % N)
    vt = api.transpose_rows(v, ld=nqb * BLOCK)
    rp_d, col_d = torch.from_numpy(row_ptr).cuda(), torch.from_numpy(col).cuda()
    order = api.schedule(rp_d, 1, 1, 1, nqb, 0, 8)
    out, lse = api.attn_fwd(q, k, vt, rp_d, col_d, BLOCK, order=order, want_lse=True, v_dim_major=True)
    torch.cuda.synchronize()
    rows = _rows(nqb)
    _compare(out, lse, host, row_ptr, col, rows, "csr")
    # the same lists as CRM rows
    W = -(-nqb // 32)
    words = np.zeros((nqb, W), dtype=np.uint32)
    for u in range(nqb):
        for c in col[row_ptr[u]:row_ptr[u + 1]]:
            words[u, c // 32] |= np.uint32(1 << (int(c) % 32))
    crm = torch.from_numpy(words.view(np.int32)).cuda()
    out2, lse2 = api.attn_fwd(q, k, vt, None, None, BLOCK, order=order, want_lse=True, v_dim_major=True, crm=crm)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(lse2, lse)
    del vt, out, out2


def test_token_sets_at_the_address_limit(big):
    q, k, v, host, _, _, _ = big
    _log("case limits N=%d (token sets)" % N)
    q_idx = np.stack([np.arange(N - 128, N), np.arange(0, 128)]).astype(np.int32)[None]      # [1][2][128]
    keys0 = np.concatenate([np.arange(N - 300, N), np.arange(0, 40)])
    keys1 = np.concatenate([np.arange(0, 64), np.arange(N - 64, N), [N + 5, -3]])
    kv_ptr = np.array([0, len(keys0), len(keys0) + len(keys1)], dtype=np.int32)
    kv_idx = np.concatenate([keys0, keys1]).astype(np.int32)
    out, lse = api.attn_tok_fwd(q, k, v, torch.from_numpy(q_idx).cuda(), torch.from_numpy(kv_ptr).cuda(),
                                torch.from_numpy(kv_idx).cuda(), want_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_tok(*host, q_idx, kv_ptr, kv_idx)
    pos = q_idx.reshape(-1).astype(np.int64)
    go = synth.bf16_bits_to_f32(out.reshape(-1, D)[torch.from_numpy(pos).cuda()].cpu().view(torch.int16)
                                .numpy().view(np.uint16)).astype(np.float64)
    gl = lse.reshape(-1)[torch.from_numpy(pos).cuda()].cpu().numpy().astype(np.float64)
    err = np.abs(go - ro)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max=float(np.abs(gl - rl).max()),
                 rows=len(pos))
    _log("  tok: %s" % stats)
    assert_within(stats)
