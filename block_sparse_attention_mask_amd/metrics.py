"""Work accounting for the metric: allowed (query, key) token pairs of a CSR.

Effective FLOPs are 4*d per allowed pair (2*d for q.k, 2*d for p*v), counting
real tokens only (positions < N) and, when causal, only s <= t.  This is the
convention behind INTRA's GFLOPS columns (4 N^2 d H dense, and N(N+1)/2
pairs per head causal, printed truncated to one decimal).
"""
from __future__ import annotations

import numpy as np


def pairs_per_entry(row_ptr: np.ndarray, col: np.ndarray, N: int, block: int, causal: bool) -> np.ndarray:
    """Allowed token pairs of every CSR entry (int64 array of len(col))."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    nqb = -(-N // block)
    R = len(row_ptr) - 1
    u = np.repeat(np.arange(R, dtype=np.int64) % nqb, np.diff(row_ptr))
    nq = np.minimum(block, N - u * block)
    nk = np.minimum(block, N - col * block)
    full = nq * nk
    if not causal:
        return full
    # diagonal block: query i (0..nq-1) sees keys 0..i of the same block
    diag = nq * (nq + 1) // 2
    return np.where(col < u, full, np.where(col == u, diag, 0))


def count_pairs(row_ptr, col, N: int, block: int, causal: bool) -> int:
    return int(pairs_per_entry(row_ptr, col, N, block, causal).sum())


def pairs_per_row(row_ptr, col, N: int, block: int, causal: bool) -> np.ndarray:
    per = pairs_per_entry(row_ptr, col, N, block, causal)
    cs = np.concatenate([[0], np.cumsum(per)])
    rp = np.asarray(row_ptr, dtype=np.int64)
    return cs[rp[1:]] - cs[rp[:-1]]


def effective_flops(row_ptr, col, N: int, block: int, d: int, causal: bool, heads_factor: int = 1) -> float:
    return 4.0 * d * count_pairs(row_ptr, col, N, block, causal) * heads_factor
