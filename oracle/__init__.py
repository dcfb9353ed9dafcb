"""CPU reference checker (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (``block_sparse_attention_mask_amd``)
never imports it.  The arithmetic lives in ``oracle.c`` (plain C, fp64,
OpenMP); this module only builds it with gcc and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

P = ctypes.c_void_p
I64 = ctypes.c_int64


# A build of oracle.c to load instead of liboracle.so (the sanitizer test
# runs the pins against an -fsanitize=address,undefined build this way).
_ALT = os.environ.get("BSA_ORACLE_LIB")


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP, -O2)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    (every finding fatal) into ``path``.  A process that loads it needs the
    ASan runtime preloaded (the Python interpreter is not instrumented)."""
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                           "-o", path, _SRC, "-lm"])
    return path


def lib():
    global _lib
    if _lib is None:
        path = _ALT or _LIB
        if not _ALT and (not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=True)
        L = ctypes.CDLL(path)
        L.oracle_build_csr.restype = I64
        L.oracle_build_csr.argtypes = [P, P, ctypes.c_float, P, I64, I64, I64, ctypes.c_int,
                                       P, P, P, I64]
        L.oracle_build_crm.restype = ctypes.c_int
        L.oracle_build_crm.argtypes = [P, P, ctypes.c_float, I64, I64, I64, ctypes.c_int, P]
        L.oracle_crm_walk.restype = I64
        L.oracle_crm_walk.argtypes = [P, I64, I64, P, P, I64]
        L.oracle_segment_offsets.restype = ctypes.c_int
        L.oracle_segment_offsets.argtypes = [P, I64, I64, ctypes.c_int32, P]
        L.oracle_segment_means.restype = ctypes.c_int
        L.oracle_segment_means.argtypes = [P, P, I64, I64, I64, I64, P, ctypes.c_int32, ctypes.c_int32, P]
        L.oracle_is_sample.restype = ctypes.c_int
        L.oracle_is_sample.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_int32, I64, ctypes.c_int32, I64,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_double, P, P, P]
        L.oracle_attn_tok.restype = ctypes.c_int
        L.oracle_attn_tok.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I64, P, P, P, ctypes.c_int,
                                      ctypes.c_double, I64, P, P, P]
        L.oracle_perm_from_labels.restype = ctypes.c_int
        L.oracle_perm_from_labels.argtypes = [P, I64, I64, ctypes.c_int32, P]
        L.oracle_schedule.restype = ctypes.c_int
        L.oracle_schedule.argtypes = [P, P, I64, I64, I64, I64, I64, I64, P, I64, P]
        L.oracle_schedule_pairs.restype = ctypes.c_int
        L.oracle_schedule_pairs.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, P, P, P]
        L.oracle_spectral_order.restype = ctypes.c_int
        L.oracle_spectral_order.argtypes = [P, P, I64, I64, I64, I64, P, P]
        L.oracle_attn_rows.restype = ctypes.c_int
        L.oracle_attn_rows.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64,
                                       P, P, P, P, P, ctypes.c_int, ctypes.c_double,
                                       I64, P, P, P]
        L.oracle_count_pairs.restype = I64
        L.oracle_count_pairs.argtypes = [P, P, I64, I64, I64, ctypes.c_int]
        L.oracle_group_mass.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, I64, P, ctypes.c_int,
                                        ctypes.c_double, I64, I64, P]
        L.oracle_group_mass.restype = ctypes.c_int
        L.oracle_topk.argtypes = [P, I64, I64, I64, P]
        L.oracle_topk.restype = ctypes.c_int
        L.oracle_stage1_decide.argtypes = [P, P, I64, I64, I64, I64, I64, I64, I64, I64, P, P, P]
        L.oracle_stage1_decide.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def build_csr(mask=None, T=None, p: float = 0.0, lw_map=None, nQB: int = 0, force_diag: bool = True,
              want_lw: bool = False):
    """Returns (row_ptr int32[R+1], col int32[nnz], lw float32[nnz] or None)."""
    src = mask if mask is not None else T
    R, nKB = src.shape
    mask = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    T = None if T is None else np.ascontiguousarray(T, dtype=np.float32)
    lw_map = None if lw_map is None else np.ascontiguousarray(lw_map, dtype=np.float32)
    row_ptr = np.zeros(R + 1, dtype=np.int32)
    n = lib().oracle_build_csr(_p(mask), _p(T), float(p), _p(lw_map), R, nQB or nKB, nKB,
                               int(force_diag), _p(row_ptr), None, None, 0)
    if n < 0:
        raise ValueError("oracle_build_csr failed: %d" % n)
    col = np.zeros(max(n, 1), dtype=np.int32)
    lw = np.zeros(max(n, 1), dtype=np.float32) if (want_lw or lw_map is not None) else None
    n2 = lib().oracle_build_csr(_p(mask), _p(T), float(p), _p(lw_map), R, nQB or nKB, nKB,
                                int(force_diag), _p(row_ptr), _p(col), _p(lw), n)
    assert n2 == n
    return row_ptr, col[:n], (None if lw is None else lw[:n])


def build_crm(mask=None, T=None, p: float = 0.0, nQB: int = 0, force_diag: bool = True):
    """Returns CRM words uint32 [R][ceil(nKB / 32)]."""
    src = mask if mask is not None else T
    R, nKB = src.shape
    mask = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    T = None if T is None else np.ascontiguousarray(T, dtype=np.float32)
    words = np.empty((R, (nKB + 31) // 32), dtype=np.uint32)
    rc = lib().oracle_build_crm(_p(mask), _p(T), float(p), R, nQB or nKB, nKB, int(force_diag),
                                _p(words))
    if rc:
        raise ValueError("oracle_build_crm failed: %d" % rc)
    return words


def crm_walk(words: np.ndarray, nKB: int):
    """Runs the CRM forward iterator over every row of ``words`` [R][W].
    Returns (row_ptr int32[R+1], col int32[nnz])."""
    words = np.ascontiguousarray(words, dtype=np.uint32)
    R, W = words.shape
    assert W == (nKB + 31) // 32
    row_ptr = np.zeros(R + 1, dtype=np.int32)
    n = lib().oracle_crm_walk(_p(words), R, nKB, _p(row_ptr), None, 0)
    if n < 0:
        raise ValueError("oracle_crm_walk failed: %d" % n)
    col = np.zeros(max(n, 1), dtype=np.int32)
    n2 = lib().oracle_crm_walk(_p(words), R, nKB, _p(row_ptr), _p(col), n)
    assert n2 == n
    return row_ptr, col[:n]


def segment_offsets(labels: np.ndarray, G: int) -> np.ndarray:
    """seg_ptr int32 [BH][G+1]: tokens of each head with label < g."""
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    BH, N = labels.shape
    sp = np.empty((BH, G + 1), dtype=np.int32)
    rc = lib().oracle_segment_offsets(_p(labels), BH, N, int(G), _p(sp))
    if rc:
        raise ValueError("oracle_segment_offsets failed: %d" % rc)
    return sp


def segment_means(x, seg_ptr=None, G: int = 0, seg_len: int = 0) -> np.ndarray:
    """x [B][H][N][d] uint16 bf16 bits (contiguous last dim).  Segments from
    seg_ptr [B*H][G+1], or fixed-length seg_len.  Returns float32 [B*H][G][d]."""
    x = np.asarray(x)
    assert x.dtype == np.uint16 and x.strides[-1] == 2
    B, H, N, d = x.shape
    if seg_ptr is not None:
        seg_ptr = np.ascontiguousarray(seg_ptr, dtype=np.int32)
        G = seg_ptr.shape[1] - 1
    else:
        G = -(-N // seg_len)
    xs = np.array([s // 2 for s in x.strides[:3]], dtype=np.int64)
    out = np.empty((B * H, G, d), dtype=np.float32)
    rc = lib().oracle_segment_means(_p(x), _p(xs), B, H, N, d, _p(seg_ptr), int(G), int(seg_len), _p(out))
    if rc:
        raise ValueError("oracle_segment_means failed: %d" % rc)
    return out


def is_sample(qbar, kbar, q_seg_ptr, uoff, B: int, Hq: int, Hkv: int, N: int, block: int, m_exact: int,
              m_sample: int, scale: Optional[float] = None):
    """Group-shared importance sampling over KV tiles.  qbar float32
    [B*Hq][G][d], kbar float32 [B*Hkv][nKB][d], q_seg_ptr int32 [B*Hq][G+1],
    uoff float64 [B*Hq][G].  Returns (mask uint8 [R][nKB], lw_map float32
    [R][nKB], pi float64 [B*Hq][G][nKB])."""
    qbar = np.ascontiguousarray(qbar, dtype=np.float32)
    kbar = np.ascontiguousarray(kbar, dtype=np.float32)
    q_seg_ptr = np.ascontiguousarray(q_seg_ptr, dtype=np.int32)
    uoff = np.ascontiguousarray(uoff, dtype=np.float64)
    G, d = qbar.shape[1], qbar.shape[2]
    nb = -(-N // block)
    assert kbar.shape == (B * Hkv, nb, d) and q_seg_ptr.shape == (B * Hq, G + 1) and uoff.shape == (B * Hq, G)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    mask = np.empty((B * Hq * nb, nb), dtype=np.uint8)
    lw = np.empty((B * Hq * nb, nb), dtype=np.float32)
    pi = np.empty((B * Hq, G, nb), dtype=np.float64)
    rc = lib().oracle_is_sample(_p(qbar), _p(kbar), _p(q_seg_ptr), _p(uoff), B, Hq, Hkv, int(G), N, int(block), d,
                                int(m_exact), int(m_sample), float(scale), _p(mask), _p(lw), _p(pi))
    if rc:
        raise ValueError("oracle_is_sample failed: %d" % rc)
    return mask, lw, pi


def perm_from_labels(labels: np.ndarray, n_clusters: int) -> np.ndarray:
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    BH, N = labels.shape
    perm = np.empty((BH, N), dtype=np.int32)
    rc = lib().oracle_perm_from_labels(_p(labels), BH, N, int(n_clusters), _p(perm))
    if rc:
        raise ValueError("oracle_perm_from_labels failed: %d" % rc)
    return perm


def schedule(row_ptr: np.ndarray, B: int, Hq: int, Hkv: int, nQB: int, W: int, n_xcd: int = 1,
             row_perm: Optional[np.ndarray] = None, head_step: int = 1, col: Optional[np.ndarray] = None):
    """Launch order of the rows; with head_step 2 only the rows of the first
    head of each pair of query heads sharing a KV head (B*Hq*nQB/2 rows).
    W = 0: buckets of 2048; with ``col`` given each keeps the sorted or the
    sequence order, whichever shares more blocks between consecutive rows."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    if col is not None:
        col = np.ascontiguousarray(col, dtype=np.int32)
    if row_perm is not None:
        row_perm = np.ascontiguousarray(row_perm, dtype=np.int32).reshape(-1)
        assert row_perm.size == B * Hq * nQB
    order = np.empty(B * Hq * nQB // head_step, dtype=np.int32)
    rc = lib().oracle_schedule(_p(row_ptr), _p(col), B, Hq, Hkv, nQB, W, n_xcd, _p(row_perm), head_step, _p(order))
    if rc:
        raise ValueError("oracle_schedule failed: %d" % rc)
    return order


def schedule_pairs(row_ptr: np.ndarray, col: np.ndarray, B: int, Hq: int, Hkv: int, nQB: int, W: int = 0,
                   n_xcd: int = 1, row_perm: Optional[np.ndarray] = None, lw: Optional[np.ndarray] = None):
    """Launch tables (order, order2) with consecutive query blocks of a head
    that list identical blocks (and log-weights) paired in one entry; the
    second row of a pair leaves an empty entry (-1, -1).  Buckets, adaptive
    order (W = 0) and XCD deal as schedule()."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    lw = None if lw is None else np.ascontiguousarray(lw, dtype=np.float32)
    if row_perm is not None:
        row_perm = np.ascontiguousarray(row_perm, dtype=np.int32).reshape(-1)
        assert row_perm.size == B * Hq * nQB
    R = B * Hq * nQB
    order = np.empty(R, dtype=np.int32)
    order2 = np.empty(R, dtype=np.int32)
    rc = lib().oracle_schedule_pairs(_p(row_ptr), _p(col), _p(lw), B, Hq, Hkv, nQB, W, n_xcd, _p(row_perm),
                                     _p(order), _p(order2))
    if rc:
        raise ValueError("oracle_schedule_pairs failed: %d" % rc)
    return order, order2


def spectral_order(row_ptr: np.ndarray, col: np.ndarray, BH: int, nQB: int, nKB: int, iters: int):
    """WaveAlign stage-1 order of every head's query blocks.  Returns
    (perm int32 [BH][nQB]: query block at each position, angle float64
    [BH][nQB]: polar angle of each query block)."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    assert row_ptr.size == BH * nQB + 1
    perm = np.empty(BH * nQB, dtype=np.int32)
    angle = np.empty(BH * nQB, dtype=np.float64)
    rc = lib().oracle_spectral_order(_p(row_ptr), _p(col), BH, nQB, nKB, iters, _p(perm), _p(angle))
    if rc:
        raise ValueError("oracle_spectral_order failed: %d" % rc)
    return perm.reshape(BH, nQB), angle.reshape(BH, nQB)


# Defaults of the stage-1 skip estimate (WaveAlign adaptive skip):
# gamma 0.04, the largest relative kernel-time reduction stage 1 gave on
# MI355X per unit of fresh-block fraction; 2.1e-3 ms per 128x128 block pair
# on one compute unit (d = 128); stage-1 cost 8.6e-4 ms per query-block row
# and 3.5e-6 ms per listed block of the largest head per 10 iterations;
# density threshold 0.10; L2 of one XCD, 4 MiB.
STAGE1_DEFAULTS = (0.04, 2.1e-3, 8.6e-4, 3.5e-6, 0.10, 4.0 * 1024 * 1024)


def stage1_decide(row_ptr, col, BH: int, nQB: int, nKB: int, N: int, d: int, block: int, iters: int,
                  n_cus: int, params=STAGE1_DEFAULTS):
    """WaveAlign's adaptive skip of stage 1.  Returns (run: bool, stats dict)."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    assert row_ptr.size == BH * nQB + 1
    prm = np.ascontiguousarray(params, dtype=np.float64)
    assert prm.size == 6
    run = np.zeros(1, dtype=np.int32)
    st = np.zeros(7, dtype=np.float64)
    rc = lib().oracle_stage1_decide(_p(row_ptr), _p(col), BH, nQB, nKB, N, d, block, iters, n_cus, _p(prm),
                                    _p(run), _p(st))
    if rc:
        raise ValueError("oracle_stage1_decide failed: %d" % rc)
    names = ("fresh_fraction", "density", "t_attn_ms", "gain_ms", "cost_ms", "kv_bytes_per_head", "run")
    return bool(run[0]), dict(zip(names, st.tolist()))


def attn_rows(q, k, v, row_ptr, col, lw, block: int, rows: np.ndarray, perm_q=None, perm_k=None,
              causal: bool = False, scale: Optional[float] = None):
    """q [B][Hq][N][d], k/v [B][Hkv][N][d] as uint16 bf16 bits (any strides with
    a contiguous last dimension).  rows: flat (b*Hq + h)*N + t, original t.
    Returns (O float64 [n][d], LSE float64 [n])."""
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    for a in (q, k, v):
        assert a.dtype == np.uint16 and a.strides[-1] == 2
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    st = lambda a: np.array([s // 2 for s in a.strides[:3]], dtype=np.int64)
    qs, ks, vs = st(q), st(k), st(v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((len(rows), d), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    lw = None if lw is None else np.ascontiguousarray(lw, dtype=np.float32)
    perm_q = None if perm_q is None else np.ascontiguousarray(perm_q, dtype=np.int32)
    perm_k = None if perm_k is None else np.ascontiguousarray(perm_k, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rc = lib().oracle_attn_rows(_p(q), _p(k), _p(v), _p(qs), _p(ks), _p(vs), B, Hq, Hkv, N, d, block,
                                _p(row_ptr), _p(col), _p(lw), _p(perm_q), _p(perm_k), int(causal),
                                float(scale), len(rows), _p(rows), _p(out), _p(lse))
    if rc:
        raise ValueError("oracle_attn_rows failed: %d" % rc)
    return out, lse


def attn_tok(q, k, v, q_idx, kv_ptr, kv_idx, slots=None, causal: bool = False, scale: Optional[float] = None):
    """Token-level attention over computational query sets.  q [B][Hq][N][d],
    k/v [B][Hkv][N][d] uint16 bf16 bits; q_idx int32 [B*Hq][C][BQ]; kv_ptr
    int32 [B*Hq*C + 1]; kv_idx int32.  slots: flat (bh*C + c)*BQ + i (all by
    default).  Returns (O float64 [n][d], LSE float64 [n]; NaN for empty
    slots)."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    for a in (q, k, v):
        assert a.dtype == np.uint16 and a.strides[-1] == 2
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    q_idx = np.ascontiguousarray(q_idx, dtype=np.int32)
    C, BQ = q_idx.shape[1], q_idx.shape[2]
    kv_ptr = np.ascontiguousarray(kv_ptr, dtype=np.int32)
    kv_idx = np.ascontiguousarray(kv_idx, dtype=np.int32)
    if kv_idx.size == 0:
        kv_idx = np.zeros(1, np.int32)
    if slots is None:
        slots = np.arange(B * Hq * C * BQ, dtype=np.int64)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    st = lambda a: np.array([s // 2 for s in a.strides[:3]], dtype=np.int64)
    out = np.empty((len(slots), d), dtype=np.float64)
    lse = np.empty(len(slots), dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rc = lib().oracle_attn_tok(_p(q), _p(k), _p(v), _p(st(q)), _p(st(k)), _p(st(v)), B, Hq, Hkv, N, d, C, BQ,
                               _p(q_idx), _p(kv_ptr), _p(kv_idx), int(causal), float(scale), len(slots), _p(slots),
                               _p(out), _p(lse))
    if rc:
        raise ValueError("oracle_attn_tok failed: %d" % rc)
    return out, lse


def count_pairs(row_ptr, col, N: int, block: int, causal: bool) -> int:
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col = np.ascontiguousarray(col, dtype=np.int32)
    n = lib().oracle_count_pairs(_p(row_ptr), _p(col), len(row_ptr) - 1, N, block, int(causal))
    if n < 0:
        raise ValueError("oracle_count_pairs failed")
    return int(n)


def attn_full(w, row_ptr, col, lw, perm_q=None, perm_k=None, rows=None):
    """Convenience: every row (or the given rows) of workload ``w``."""
    if rows is None:
        rows = np.arange(w.B * w.Hq * w.N, dtype=np.int64)
    return attn_rows(w.q, w.k, w.v, row_ptr, col, lw, w.block, rows, perm_q, perm_k, w.causal)


def group_mass(q, k, q_idx, causal: bool = False, scale: Optional[float] = None, keys=None):
    """MC-Sparse's exact selection, second pass: per query group (q_idx int32
    [B*Hq][C][BQ], empty slots outside [0, N)), the sum over the group's
    queries of each key's attention probability under the dense softmax
    (causal: keys after the query excluded).  keys = (s0, s1) restricts the
    output columns.  Returns float64 [B*Hq*C][s1 - s0]."""
    q, k = np.asarray(q), np.asarray(k)
    for a in (q, k):
        assert a.dtype == np.uint16 and a.strides[-1] == 2
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    q_idx = np.ascontiguousarray(q_idx, dtype=np.int32)
    C, BQ = q_idx.shape[1], q_idx.shape[2]
    s0, s1 = (0, N) if keys is None else keys
    st = lambda a: np.array([s // 2 for s in a.strides[:3]], dtype=np.int64)
    out = np.empty((B * Hq * C, s1 - s0), dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rc = lib().oracle_group_mass(_p(q), _p(k), _p(st(q)), _p(st(k)), B, Hq, Hkv, N, d, C, BQ, _p(q_idx),
                                 int(causal), float(scale), int(s0), int(s1), _p(out))
    if rc:
        raise ValueError("oracle_group_mass failed: %d" % rc)
    return out


def topk(mass, K: int) -> np.ndarray:
    """The K largest of each row (ties to the lower index), ascending indices:
    int32 [rows][min(K, N)].  float32 input is widened exactly."""
    mass = np.ascontiguousarray(np.asarray(mass, dtype=np.float64))
    rows, N = mass.shape
    k = min(K, N)
    idx = np.empty((rows, k), dtype=np.int32)
    rc = lib().oracle_topk(_p(mass), rows, N, int(K), _p(idx))
    if rc:
        raise ValueError("oracle_topk failed: %d" % rc)
    return idx
