"""Python binding of libbsattn.so.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory (tensors) and the stream
(``torch.cuda.current_stream()``).  bf16 tensors may be ``torch.bfloat16`` or
``torch.uint16``/``int16`` holding bf16 bit patterns; the head dimension must
be contiguous.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import AttnArgs, I64, I64x3, MassArgs, Stage1Params, TokArgs, check, load

__all__ = ["version", "csr_count", "csr_fill", "build_csr", "perm_from_labels", "permute_rows",
           "unpermute_rows", "transpose_rows", "schedule", "attn_fwd", "device_cus", "crm_build",
           "crm_row_ptr", "crm_to_csr", "segment_offsets", "segment_means", "is_sample",
           "attn_tok_fwd"]

_BF16_LIKE = (torch.bfloat16, torch.uint16, torch.int16)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError("%s has dtype %s" % (name, t.dtype))
    return t


def _strides(t: torch.Tensor) -> I64x3:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B][H][N][d] tensor with contiguous last dimension")
    return I64x3(t.stride(0), t.stride(1), t.stride(2))


def version() -> int:
    return load().bsa_version()


def device_cus() -> int:
    n = load().bsa_device_cus()
    if n < 0:
        check("bsa_device_cus", n)
    return n


def device_clock_khz() -> int:
    k = load().bsa_device_clock_khz()
    if k < 0:
        check("bsa_device_clock_khz", k)
    return k


def clock_under_mfma_load(blocks: int = 0, iters: int = 40000, random_operands: bool = False,
                          stream=None) -> dict:
    """bsa_clock_probe over every CU (2 workgroups per CU by default, so that
    every wavefront is resident from start to end):
    median, min and max engine clock in MHz of the wavefronts, and the MFMA
    rate of the launch in TFLOP/s (HIP events around it on its stream).  With
    ``random_operands`` every MFMA sees new random bf16 operands."""
    if blocks <= 0:
        blocks = 2 * device_cus()
    ticks = torch.zeros(4 * blocks * 2, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream() if stream is None else stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    check("bsa_clock_probe", load().bsa_clock_probe(int(blocks), int(iters), int(bool(random_operands)),
                                                    _ptr(ticks), _stream(s)))
    e1.record(s)
    torch.cuda.synchronize()
    t = ticks.cpu().numpy().reshape(-1, 2).astype("float64")
    mhz = sorted(t[:, 0] / t[:, 1] * 100.0)
    flop = 4.0 * iters * 32768.0 * 4 * blocks
    return {"median": round(mhz[len(mhz) // 2], 1), "min": round(mhz[0], 1), "max": round(mhz[-1], 1),
            "tflops": round(flop / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)}


def csr_count(mask=None, T=None, p: float = 0.0, nQB: Optional[int] = None, force_diag: bool = True,
              row_ptr: Optional[torch.Tensor] = None, want_nnz: bool = True,
              stream=None) -> Tuple[torch.Tensor, Optional[int]]:
    """bsa_csr_count -> (row_ptr, nnz); with want_nnz=False no host round trip
    and nnz is None."""
    src = mask if mask is not None else T
    R, nKB = src.shape
    nQB = nKB if nQB is None else nQB
    if mask is not None:
        _dev(mask, "mask", torch.uint8)
    if T is not None:
        _dev(T, "T", torch.float32)
    if not src.is_contiguous():
        raise ValueError("mask / T must be contiguous [R][nKB]")
    if row_ptr is None:
        row_ptr = torch.empty(R + 1, dtype=torch.int32, device=src.device)
    nnz = I64(0)
    check("bsa_csr_count", load().bsa_csr_count(_ptr(mask), _ptr(T), float(p), R, nQB, nKB,
                                                int(force_diag), _ptr(row_ptr),
                                                ctypes.byref(nnz) if want_nnz else None, _stream(stream)))
    return row_ptr, (int(nnz.value) if want_nnz else None)


def csr_fill(row_ptr: torch.Tensor, nnz: int, mask=None, T=None, p: float = 0.0, lw_map=None,
             nQB: Optional[int] = None, force_diag: bool = True, want_lw: bool = False,
             col=None, lw=None, stream=None):
    src = mask if mask is not None else T
    R, nKB = src.shape
    nQB = nKB if nQB is None else nQB
    dev = src.device
    if col is None:
        col = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)
    if lw is None and (want_lw or lw_map is not None):
        lw = torch.empty(max(nnz, 1), dtype=torch.float32, device=dev)
    if lw_map is not None:
        _dev(lw_map, "lw_map", torch.float32)
    check("bsa_csr_fill", load().bsa_csr_fill(_ptr(mask), _ptr(T), float(p), _ptr(lw_map), R, nQB, nKB,
                                              int(force_diag), _ptr(row_ptr), _ptr(col), _ptr(lw),
                                              col.numel(), _stream(stream)))
    return col[:nnz], (None if lw is None else lw[:nnz])


def build_csr(mask=None, T=None, p: float = 0.0, lw_map=None, nQB: Optional[int] = None,
              force_diag: bool = True, want_lw: bool = False, sync: bool = True, stream=None):
    """bsa_csr_count + allocation + bsa_csr_fill -> (row_ptr, col, lw or None).
    With sync=False, col (and lw) are sized by the bound R * nKB, so no host
    round trip is needed; entries past row_ptr[R] are unused."""
    if sync:
        row_ptr, nnz = csr_count(mask, T, p, nQB, force_diag, stream=stream)
    else:
        row_ptr, _ = csr_count(mask, T, p, nQB, force_diag, want_nnz=False, stream=stream)
        src = mask if mask is not None else T
        nnz = src.shape[0] * src.shape[1]
    col, lw = csr_fill(row_ptr, nnz, mask, T, p, lw_map, nQB, force_diag, want_lw, stream=stream)
    return row_ptr, col, lw


def crm_build(mask=None, T=None, p: float = 0.0, nQB: Optional[int] = None, force_diag: bool = True,
              crm: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bsa_crm_build -> CRM rows, int32 [R][ceil(nKB / 32)] holding the uint32 words."""
    src = mask if mask is not None else T
    R, nKB = src.shape
    nQB = nKB if nQB is None else nQB
    if mask is not None:
        _dev(mask, "mask", torch.uint8)
    if T is not None:
        _dev(T, "T", torch.float32)
    if not src.is_contiguous():
        raise ValueError("mask / T must be contiguous [R][nKB]")
    W = (nKB + 31) // 32
    if crm is None:
        crm = torch.empty((R, W), dtype=torch.int32, device=src.device)
    elif crm.numel() < R * W or not crm.is_contiguous():
        raise ValueError("crm must be a contiguous buffer of R * ceil(nKB / 32) words")
    check("bsa_crm_build", load().bsa_crm_build(_ptr(mask), _ptr(T), float(p), R, nQB, nKB, int(force_diag),
                                                _ptr(crm), _stream(stream)))
    return crm


def _crm_rows(crm: torch.Tensor, nKB: int) -> int:
    _dev(crm, "crm", (torch.int32, torch.uint32))
    W = (nKB + 31) // 32
    if not crm.is_contiguous() or crm.numel() % W:
        raise ValueError("crm must be contiguous [R][ceil(nKB / 32)]")
    return crm.numel() // W


def crm_row_ptr(crm: torch.Tensor, nKB: int, row_ptr: Optional[torch.Tensor] = None, want_nnz: bool = True,
                stream=None):
    """bsa_crm_row_ptr -> (row_ptr int32 [R+1], nnz or None)."""
    R = _crm_rows(crm, nKB)
    if row_ptr is None:
        row_ptr = torch.empty(R + 1, dtype=torch.int32, device=crm.device)
    nnz = I64(0)
    check("bsa_crm_row_ptr", load().bsa_crm_row_ptr(_ptr(crm), R, nKB, _ptr(row_ptr),
                                                    ctypes.byref(nnz) if want_nnz else None, _stream(stream)))
    return row_ptr, (int(nnz.value) if want_nnz else None)


def crm_to_csr(crm: torch.Tensor, nKB: int, row_ptr: torch.Tensor, nnz: int, col=None, stream=None):
    """bsa_crm_to_csr -> col int32 [nnz] (ascending per row)."""
    R = _crm_rows(crm, nKB)
    if col is None:
        col = torch.empty(max(nnz, 1), dtype=torch.int32, device=crm.device)
    check("bsa_crm_to_csr", load().bsa_crm_to_csr(_ptr(crm), R, nKB, _ptr(row_ptr), _ptr(col), col.numel(),
                                                  _stream(stream)))
    return col[:nnz]


def segment_offsets(labels: torch.Tensor, G: int, seg_ptr: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """bsa_segment_offsets -> int32 [BH][G+1]."""
    _dev(labels, "labels", torch.int32)
    if labels.dim() != 2 or not labels.is_contiguous():
        raise ValueError("labels must be contiguous [BH][N]")
    BH, N = labels.shape
    if seg_ptr is None:
        seg_ptr = torch.empty((BH, G + 1), dtype=torch.int32, device=labels.device)
    check("bsa_segment_offsets", load().bsa_segment_offsets(_ptr(labels), BH, N, int(G), _ptr(seg_ptr),
                                                            _stream(stream)))
    return seg_ptr


def segment_means(x: torch.Tensor, seg_ptr: Optional[torch.Tensor] = None, seg_len: int = 0,
                  means: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bsa_segment_means -> float32 [B*H][G][d]; segments from seg_ptr [B*H][G+1]
    or of fixed length seg_len."""
    _dev(x, "x", _BF16_LIKE)
    B, H, N, d = x.shape
    if seg_ptr is not None:
        _dev(seg_ptr, "seg_ptr", torch.int32)
        if seg_ptr.shape != (B * H, seg_ptr.shape[1]) or not seg_ptr.is_contiguous():
            raise ValueError("seg_ptr must be contiguous [B*H][G+1]")
        G = seg_ptr.shape[1] - 1
    else:
        G = -(-N // seg_len)
    if means is None:
        means = torch.empty((B * H, G, d), dtype=torch.float32, device=x.device)
    check("bsa_segment_means", load().bsa_segment_means(_ptr(x), _strides(x), B, H, N, d, _ptr(seg_ptr), int(G),
                                                        int(seg_len), _ptr(means), _stream(stream)))
    return means


def is_sample(qbar: torch.Tensor, kbar: torch.Tensor, q_seg_ptr: torch.Tensor, uoff: torch.Tensor, B: int, Hq: int,
              Hkv: int, N: int, block: int, m_exact: int, m_sample: int, scale: float = 0.0, want_pi: bool = False,
              mask=None, lw_map=None, stream=None):
    """bsa_is_sample -> (mask uint8 [B*Hq*nKB][nKB], lw_map float32, pi float64 [B*Hq][G][nKB] or None)."""
    _dev(qbar, "qbar", torch.float32)
    _dev(kbar, "kbar", torch.float32)
    _dev(q_seg_ptr, "q_seg_ptr", torch.int32)
    _dev(uoff, "uoff", torch.float64)
    G, d = qbar.shape[1], qbar.shape[2]
    nb = -(-N // block)
    if (qbar.shape != (B * Hq, G, d) or kbar.shape != (B * Hkv, nb, d) or q_seg_ptr.shape != (B * Hq, G + 1)
            or uoff.shape != (B * Hq, G)):
        raise ValueError("qbar [B*Hq][G][d], kbar [B*Hkv][nKB][d], q_seg_ptr [B*Hq][G+1], uoff [B*Hq][G]")
    for t in (qbar, kbar, q_seg_ptr, uoff):
        if not t.is_contiguous():
            raise ValueError("sampler inputs must be contiguous")
    dev = qbar.device
    if mask is None:
        mask = torch.empty((B * Hq * nb, nb), dtype=torch.uint8, device=dev)
    if lw_map is None:
        lw_map = torch.empty((B * Hq * nb, nb), dtype=torch.float32, device=dev)
    pi = torch.empty((B * Hq, G, nb), dtype=torch.float64, device=dev) if want_pi else None
    check("bsa_is_sample", load().bsa_is_sample(_ptr(qbar), _ptr(kbar), _ptr(q_seg_ptr), _ptr(uoff), B, Hq, Hkv,
                                                int(G), N, int(block), d, int(m_exact), int(m_sample), float(scale),
                                                _ptr(mask), _ptr(lw_map), _ptr(pi), _stream(stream)))
    return mask, lw_map, pi


def perm_from_labels(labels: torch.Tensor, n_clusters: int, perm=None, stream=None) -> torch.Tensor:
    _dev(labels, "labels", torch.int32)
    labels = labels.contiguous()
    BH, N = labels.shape
    if perm is None:
        perm = torch.empty_like(labels)
    check("bsa_perm_from_labels", load().bsa_perm_from_labels(_ptr(labels), BH, N, int(n_clusters),
                                                              _ptr(perm), _stream(stream)))
    return perm


def _permute(fn_name: str, src: torch.Tensor, perm: torch.Tensor, dst=None, stream=None):
    _dev(src, "src", _BF16_LIKE)
    _dev(perm, "perm", torch.int32)
    B, H, N, d = src.shape
    if dst is None:
        dst = torch.empty_like(src, memory_format=torch.contiguous_format)
    fn = getattr(load(), fn_name)
    check(fn_name, fn(_ptr(src), _ptr(dst), _ptr(perm.contiguous()), B, H, N, d, _strides(src),
                      _strides(dst), _stream(stream)))
    return dst


def permute_rows(src, perm, dst=None, stream=None):
    """dst[b][h][i] = src[b][h][perm[b*H + h][i]]."""
    return _permute("bsa_permute_rows", src, perm, dst, stream)


def unpermute_rows(src, perm, dst=None, stream=None):
    """dst[b][h][perm[b*H + h][i]] = src[b][h][i]."""
    return _permute("bsa_unpermute_rows", src, perm, dst, stream)


def transpose_rows(src: torch.Tensor, perm: Optional[torch.Tensor] = None, ld: Optional[int] = None,
                   dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dst[b][h][c][i] = src[b][h][perm[b*H + h][i] (or i)][c] for i < N, zeros
    for N <= i < ld: the dim-major V the attention kernel reads."""
    _dev(src, "src", _BF16_LIKE)
    B, H, N, d = src.shape
    if ld is None:
        ld = -(-N // 128) * 128
    if dst is None:
        dst = torch.empty((B, H, d, ld), dtype=src.dtype, device=src.device)
    if perm is not None:
        _dev(perm, "perm", torch.int32)
        perm = perm.contiguous()
    check("bsa_transpose_rows", load().bsa_transpose_rows(_ptr(src), _ptr(dst), _ptr(perm), B, H, N, d, int(ld),
                                                          _strides(src), _strides(dst), _stream(stream)))
    return dst


def schedule(row_ptr: torch.Tensor, B: int, Hq: int, Hkv: int, nQB: int, wave_rows: int = 0,
             n_xcd: int = 8, order=None, stream=None, row_perm: Optional[torch.Tensor] = None,
             head_step: int = 1, col: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Launch order of the attention rows; head_step 2 lists one row per pair
    of query heads sharing a KV head (for attn_fwd(kv_share=True)).  With
    wave_rows 0 and the block lists ``col``, each segment keeps the sorted or
    the sequence order, whichever shares more blocks between consecutive
    rows."""
    _dev(row_ptr, "row_ptr", torch.int32)
    if col is not None:
        _dev(col, "col", torch.int32)
    if row_perm is not None:
        _dev(row_perm, "row_perm", torch.int32)
        if row_perm.numel() != B * Hq * nQB:
            raise ValueError("row_perm must hold B*Hq*nQB entries")
    if order is None:
        order = torch.empty(B * Hq * nQB // head_step, dtype=torch.int32, device=row_ptr.device)
    check("bsa_schedule", load().bsa_schedule(_ptr(row_ptr), _ptr(col), B, Hq, Hkv, nQB, int(wave_rows), int(n_xcd),
                                              _ptr(row_perm), int(head_step), _ptr(order), _stream(stream)))
    return order


def schedule_pairs(row_ptr: torch.Tensor, col: torch.Tensor, B: int, Hq: int, Hkv: int, nQB: int,
                   wave_rows: int = 0, n_xcd: int = 8, lw: Optional[torch.Tensor] = None,
                   row_perm: Optional[torch.Tensor] = None, stream=None):
    """Launch tables (order, order2) for attn_fwd(order=..., order2=...):
    consecutive query blocks of a head whose lists (and log-weights) are
    identical share one entry; the second row of a pair leaves an empty entry
    (-1, -1) at the end of its bucket.  Buckets and order as schedule()."""
    _dev(row_ptr, "row_ptr", torch.int32)
    _dev(col, "col", torch.int32)
    if lw is not None:
        _dev(lw, "lw", torch.float32)
    if row_perm is not None:
        _dev(row_perm, "row_perm", torch.int32)
        if row_perm.numel() != B * Hq * nQB:
            raise ValueError("row_perm must hold B*Hq*nQB entries")
    order = torch.empty(B * Hq * nQB, dtype=torch.int32, device=row_ptr.device)
    order2 = torch.empty_like(order)
    check("bsa_schedule_pairs", load().bsa_schedule_pairs(_ptr(row_ptr), _ptr(col), _ptr(lw), B, Hq, Hkv, nQB,
                                                          int(wave_rows), int(n_xcd), _ptr(row_perm),
                                                          _ptr(order), _ptr(order2), _stream(stream)))
    return order, order2


def pair_rows_equal(row_ptr: torch.Tensor, col: torch.Tensor, B: int, Hq: int, Hkv: int, nQB: int,
                    lw: Optional[torch.Tensor] = None, equal: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Device int32 [1]: 1 if the rows of query heads 2j and 2j + 1 of every
    KV group are identical (lists and log-weights), the precondition of
    attn_fwd(kv_share=True); else 0."""
    _dev(row_ptr, "row_ptr", torch.int32)
    _dev(col, "col", torch.int32)
    if lw is not None:
        _dev(lw, "lw", torch.float32)
    if row_ptr.numel() != B * Hq * nQB + 1:
        raise ValueError("row_ptr must hold B*Hq*nQB + 1 entries")
    if equal is None:
        equal = torch.empty(1, dtype=torch.int32, device=row_ptr.device)
    check("bsa_pair_rows_equal", load().bsa_pair_rows_equal(_ptr(row_ptr), _ptr(col), _ptr(lw), B, Hq, Hkv, nQB,
                                                            _ptr(equal), _stream(stream)))
    return equal


def spectral_order(row_ptr: torch.Tensor, col: torch.Tensor, BH: int, nQB: int, nKB: int, iters: int = 10,
                   want_angle: bool = False, enable: Optional[torch.Tensor] = None, stream=None):
    """WaveAlign stage-1 order of every head's query blocks: (perm int32
    [BH][nQB], angle float64 [BH][nQB] or None).  With ``enable`` (device
    int32 [1], e.g. stage1_decide's decision) holding 0 the order is the
    identity and nothing is computed."""
    _dev(row_ptr, "row_ptr", torch.int32)
    _dev(col, "col", torch.int32)
    if enable is not None:
        _dev(enable, "enable", torch.int32)
    if row_ptr.numel() != BH * nQB + 1:
        raise ValueError("row_ptr must hold BH*nQB + 1 entries")
    perm = torch.empty((BH, nQB), dtype=torch.int32, device=row_ptr.device)
    angle = torch.empty((BH, nQB), dtype=torch.float64, device=row_ptr.device) if want_angle else None
    check("bsa_spectral_order", load().bsa_spectral_order(_ptr(row_ptr), _ptr(col), BH, nQB, nKB, int(iters),
                                                          _ptr(perm), _ptr(angle), _ptr(enable),
                                                          _stream(stream)))
    return perm, angle


def spectral_supported(nQB: int, nKB: int) -> bool:
    """The shapes bsa_spectral_order accepts (its LDS bitmask limits)."""
    return (nQB <= 1024 and nKB <= 1024 and nKB * ((nQB + 31) // 32) <= 12288
            and nQB * ((nKB + 31) // 32) <= 12288)


STAGE1_PARAM_NAMES = ("gamma", "tile_ms", "row_ms", "nnz_ms", "density_min", "l2_bytes")
STAGE1_STAT_NAMES = ("fresh_fraction", "density", "t_attn_ms", "gain_ms", "cost_ms", "kv_bytes_per_head", "run")


def stage1_default_params() -> dict:
    p = Stage1Params()
    load().bsa_stage1_default_params(ctypes.byref(p))
    return {n: getattr(p, n) for n in STAGE1_PARAM_NAMES}


def stage1_decide(row_ptr: torch.Tensor, col: torch.Tensor, BH: int, nQB: int, nKB: int, N: int, d: int,
                  block: int, iters: int = 10, n_cus: int = 0, params: Optional[dict] = None, stream=None):
    """WaveAlign's adaptive skip: (decision int32 [1], stats float64 [7]),
    both on the device (no synchronisation).  n_cus = 0: the device's
    compute units.  params: overrides of stage1_default_params()."""
    _dev(row_ptr, "row_ptr", torch.int32)
    _dev(col, "col", torch.int32)
    if row_ptr.numel() != BH * nQB + 1:
        raise ValueError("row_ptr must hold BH*nQB + 1 entries")
    prm = None
    if params is not None:
        vals = stage1_default_params()
        vals.update(params)
        prm = Stage1Params(*[float(vals[n]) for n in STAGE1_PARAM_NAMES])
    dec = torch.empty(1, dtype=torch.int32, device=row_ptr.device)
    stats = torch.empty(7, dtype=torch.float64, device=row_ptr.device)
    cus = int(n_cus) if n_cus else device_cus()
    check("bsa_stage1_decide", load().bsa_stage1_decide(_ptr(row_ptr), _ptr(col), BH, nQB, nKB, int(N), int(d),
                                                        int(block), int(iters), cus,
                                                        ctypes.byref(prm) if prm is not None else None,
                                                        _ptr(dec), _ptr(stats), _stream(stream)))
    return dec, stats


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, row_ptr: Optional[torch.Tensor],
             col: Optional[torch.Tensor], block: int, lw: Optional[torch.Tensor] = None,
             order: Optional[torch.Tensor] = None, scatter_perm_q: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             want_lse: bool = False, scale: float = 0.0, causal: bool = False,
             v_dim_major: bool = False, crm: Optional[torch.Tensor] = None,
             gather_perm_q: Optional[torch.Tensor] = None, kv_share: bool = False,
             order2: Optional[torch.Tensor] = None, stream=None):
    """Block-sparse attention forward; returns (out, lse or None).  With
    ``v_dim_major`` v is [B][Hkv][d][ld] (keys contiguous, from transpose_rows),
    otherwise [B][Hkv][N][d].  With ``crm`` (CRM rows from crm_build) the lists
    come from the bitmask words and row_ptr/col may be None.  With
    ``gather_perm_q`` q is unpermuted and the kernel reads query row
    gather_perm_q[bh][i] for permuted position i.  With ``kv_share`` the rows
    of query heads 2j and 2j + 1 of every KV group must be identical
    (pair_rows_equal checks it): one launch serves both, and order, if given,
    comes from schedule(..., head_step=2).  With ``order2`` (beside order,
    same length) launch entry i also serves row order2[i] when it is a row:
    the two rows list identical blocks (schedule_pairs builds such tables)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, _BF16_LIKE)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B * Hq, N), dtype=torch.float32, device=q.device)
    a = AttnArgs()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)
    a.B, a.Hq, a.Hkv, a.d, a.block, a.N = B, Hq, Hkv, d, int(block), N
    a.q_str, a.k_str, a.v_str, a.o_str = _strides(q), _strides(k), _strides(v), _strides(out)
    a.row_ptr, a.col = _ptr(row_ptr), _ptr(col)
    a.lw = _ptr(lw)
    a.order = _ptr(order)
    a.n_order = 0 if order is None else order.numel()
    a.scatter_perm_q = _ptr(scatter_perm_q)
    a.scale = float(scale)
    a.causal = int(bool(causal))
    a.v_layout = _lib.BSA_V_DIM_MAJOR if v_dim_major else _lib.BSA_V_TOKEN_MAJOR
    if crm is not None:
        nQB = -(-N // int(block))
        if _crm_rows(crm, nQB) != B * Hq * nQB:
            raise ValueError("crm must hold B * Hq * ceil(N / block) rows")
    a.crm = _ptr(crm)
    a.gather_perm_q = _ptr(gather_perm_q)
    a.kv_share = 2 if kv_share else 0
    if order2 is not None:
        _dev(order2, "order2", (torch.int32,))
        if order is None or order2.numel() != order.numel():
            raise ValueError("order2 needs order, with as many entries")
    a.order2 = _ptr(order2)
    check("bsa_attn_fwd", load().bsa_attn_fwd(ctypes.byref(a), _stream(stream)))
    return out, lse


def attn_tok_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_idx: torch.Tensor, kv_ptr: torch.Tensor,
                 kv_idx: torch.Tensor, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 want_lse: bool = False, scale: float = 0.0, causal: bool = False, kv_share=False,
                 stream=None):
    """Token-level attention over computational query sets: q_idx int32
    [B*Hq][n_sets][set_size] query positions, kv_ptr int32 [B*Hq*n_sets + 1]
    and kv_idx int32 key positions; q, k, v token-major.  Returns (out, lse).
    Rows of out at positions no set lists are left as they were (out is
    zero-filled when allocated here).  With ``kv_share`` (True or 2, or 4)
    the sets of each run of 2 (or 4) consecutive query heads of a KV group
    must be identical: one launch serves them all, gathering each K/V tile
    once for them."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, _BF16_LIKE)
    for t, n in ((q_idx, "q_idx"), (kv_ptr, "kv_ptr"), (kv_idx, "kv_idx")):
        _dev(t, n, torch.int32)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % n)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if q_idx.dim() != 3 or q_idx.shape[0] != B * Hq:
        raise ValueError("q_idx must be [B*Hq][n_sets][set_size]")
    n_sets, set_size = q_idx.shape[1], q_idx.shape[2]
    if kv_ptr.numel() != B * Hq * n_sets + 1:
        raise ValueError("kv_ptr must have B*Hq*n_sets + 1 entries")
    if out is None:
        out = torch.zeros((B, Hq, N, d), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.full((B * Hq, N), float("nan"), dtype=torch.float32, device=q.device)
    a = TokArgs()
    a.q, a.k, a.v, a.o, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)
    a.B, a.Hq, a.Hkv, a.d, a.N = B, Hq, Hkv, d, N
    a.q_str, a.k_str, a.v_str, a.o_str = _strides(q), _strides(k), _strides(v), _strides(out)
    a.n_sets, a.set_size = n_sets, set_size
    a.q_idx, a.kv_ptr, a.kv_idx = _ptr(q_idx), _ptr(kv_ptr), _ptr(kv_idx)
    a.scale = float(scale)
    a.causal = int(bool(causal))
    a.kv_share = 0 if not kv_share else (2 if kv_share is True else int(kv_share))
    check("bsa_attn_tok_fwd", load().bsa_attn_tok_fwd(ctypes.byref(a), _stream(stream)))
    return out, lse


def group_mass(q: torch.Tensor, k: torch.Tensor, lse: torch.Tensor, q_idx: torch.Tensor, keys=None,
               out: Optional[torch.Tensor] = None, scale: float = 0.0, causal: bool = False, stream=None):
    """Exact KV selection, mass pass: for each query set (q_idx int32
    [B*Hq][n_sets][set_size]) and key s in keys = (k0, k1) (default all), the
    sum over the set's queries of exp(q_t . k_s * scale - lse_t), lse float32
    [B*Hq][N] from the dense pass.  Returns float32 [B*Hq*n_sets][k1 - k0]."""
    for t, n in ((q, "q"), (k, "k")):
        _dev(t, n, _BF16_LIKE)
    _dev(lse, "lse", torch.float32)
    _dev(q_idx, "q_idx", torch.int32)
    if not lse.is_contiguous() or not q_idx.is_contiguous():
        raise ValueError("lse and q_idx must be contiguous")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if q_idx.dim() != 3 or q_idx.shape[0] != B * Hq:
        raise ValueError("q_idx must be [B*Hq][n_sets][set_size]")
    if lse.shape != (B * Hq, N):
        raise ValueError("lse must be [B*Hq][N]")
    n_sets, set_size = q_idx.shape[1], q_idx.shape[2]
    k0, k1 = (0, N) if keys is None else keys
    shape = (B * Hq * n_sets, k1 - k0)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != shape or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 %s" % (shape,))
    a = MassArgs()
    a.q, a.k, a.lse, a.mass = _ptr(q), _ptr(k), _ptr(lse), _ptr(out)
    a.B, a.Hq, a.Hkv, a.d, a.N = B, Hq, Hkv, d, N
    a.q_str, a.k_str = _strides(q), _strides(k)
    a.n_sets, a.set_size = n_sets, set_size
    a.q_idx = _ptr(q_idx)
    a.k0, a.k1 = int(k0), int(k1)
    a.scale = float(scale)
    a.causal = int(bool(causal))
    check("bsa_group_mass", load().bsa_group_mass(ctypes.byref(a), _stream(stream)))
    return out


def topk_rows(x: torch.Tensor, k: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Column indices of the k largest values of each row of x (float32
    [rows][n], unit column stride), ties to the lower index, ascending:
    int32 [rows][min(k, n)]."""
    _dev(x, "x", torch.float32)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [rows][n] with unit column stride")
    rows, n = x.shape
    kk = min(int(k), n)
    if out is None:
        out = torch.empty((rows, kk), dtype=torch.int32, device=x.device)
    elif out.dtype != torch.int32 or tuple(out.shape) != (rows, kk) or not out.is_contiguous():
        raise ValueError("out must be contiguous int32 [rows][min(k, n)]")
    check("bsa_topk_rows", load().bsa_topk_rows(_ptr(x), rows, n, x.stride(0), int(k), _ptr(out),
                                                _stream(stream)))
    return out
