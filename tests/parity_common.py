"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from block_sparse_attention_mask_amd import pipeline
import synth

# bf16 inputs, fp32 accumulation, P and O rounded to bf16.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def bf16_tensor_to_f32(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits_to_f32(t.cpu().numpy().view(np.uint16))


def oracle_csr(w):
    return oracle.build_csr(w.mask, w.T, w.p, w.lw_map, w.nQB, w.force_diag)


def oracle_perms(w):
    if not w.permuted:
        return None, None
    return (oracle.perm_from_labels(w.labels_q, w.n_clusters),
            oracle.perm_from_labels(w.labels_k, w.n_clusters))


def sample_rows(w, seed: int = 0, per_block: bool = True) -> np.ndarray:
    """Flat (b*Hq + h)*N + t rows, t in original order: for every (b, h, query
    block) the first and last real row of the block in the sequence the kernel
    sees (permuted when there is a permutation: mapped back through perm_q), and
    per (b, h) one random whole block plus the whole tail block."""
    rng = np.random.default_rng(seed)
    nb = w.nQB
    rows = []
    perm_q, _ = oracle_perms(w)
    for bh in range(w.B * w.Hq):
        pos = []
        if per_block:
            firsts = np.arange(nb) * w.block
            lasts = np.minimum(firsts + w.block, w.N) - 1
            pos += [firsts, lasts]
        rb = int(rng.integers(0, nb))
        pos.append(np.arange(rb * w.block, min(w.N, (rb + 1) * w.block)))
        pos.append(np.arange((nb - 1) * w.block, w.N))
        p = np.unique(np.concatenate(pos))
        t = perm_q[bh][p] if perm_q is not None else p
        rows.append(bh * w.N + t.astype(np.int64))
    return np.unique(np.concatenate(rows))


def run_gpu(w, **kw):
    dw = pipeline.to_device(w)
    res = pipeline.forward(dw, want_lse=True, **kw)
    torch.cuda.synchronize()
    return dw, res


def compare_rows(w, res, rows, perm_q=None, perm_k=None, csr=None):
    if csr is None:
        csr = oracle_csr(w)
    rp, col, lw = csr
    ref_o, ref_l = oracle.attn_rows(w.q, w.k, w.v, rp, col, lw, w.block, rows, perm_q, perm_k, w.causal)
    out = bf16_tensor_to_f32(res.out).reshape(-1, w.d)[rows].astype(np.float64)
    lse = res.lse.cpu().numpy().reshape(-1)[rows].astype(np.float64)
    err = np.abs(out - ref_o)
    finite = np.isfinite(ref_l)
    lerr = np.abs(lse[finite] - ref_l[finite]) if finite.any() else np.zeros(1)
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), lse_max=float(lerr.max()),
                 rows=int(len(rows)))
    assert np.all(np.isneginf(lse[~finite])), "empty rows must have LSE = -inf"
    return stats


def assert_within(stats):
    assert stats["max_abs"] <= MAX_ABS, stats
    assert stats["mean_abs"] <= MEAN_ABS, stats
    assert stats["lse_max"] <= LSE_ABS, stats
