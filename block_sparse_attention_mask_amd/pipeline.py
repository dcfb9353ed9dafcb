"""One pass of the whole block-sparse attention path on device tensors:

mask / threshold map -> CSR (bsa_csr_count, bsa_csr_fill), or CRM rows
   (bsa_crm_build) with row offsets from their popcounts (bsa_crm_row_ptr);
   or, with a sampler, the mask and log-weights drawn on the device
   (bsa_segment_offsets, bsa_segment_means, bsa_is_sample) before the CSR
-> [cluster labels -> permutations; gather K (Q's gather is fused into the
   attention kernel's load, or done by bsa_permute_rows)]   (permuted workloads)
-> V gathered (when permuted) and written dim-major (bsa_transpose_rows)
-> row schedule (bsa_schedule)
-> attention forward (bsa_attn_fwd), with the inverse query permutation fused
   into the output store, or applied by bsa_unpermute_rows.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import api


@dataclass
class DeviceWorkload:
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    block: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    mask: Optional[torch.Tensor] = None
    T: Optional[torch.Tensor] = None
    p: float = 0.0
    lw_map: Optional[torch.Tensor] = None
    labels_q: Optional[torch.Tensor] = None
    labels_k: Optional[torch.Tensor] = None
    n_clusters: int = 0
    causal: bool = False
    force_diag: bool = True

    @property
    def nQB(self) -> int:
        return -(-self.N // self.block)

    @property
    def permuted(self) -> bool:
        return self.labels_q is not None


def to_device(w, device="cuda") -> DeviceWorkload:
    """Copy a host workload (numpy arrays of bf16 bits etc.) to device tensors."""
    t = lambda a, dt=None: None if a is None else torch.from_numpy(
        np.ascontiguousarray(a if dt is None else a.view(dt))).to(device)
    return DeviceWorkload(w.B, w.Hq, w.Hkv, w.N, w.d, w.block,
                          t(w.q, np.int16), t(w.k, np.int16), t(w.v, np.int16),
                          t(w.mask), t(w.T), float(w.p), t(w.lw_map), t(w.labels_q), t(w.labels_k),
                          int(w.n_clusters), bool(w.causal), bool(w.force_diag))


_side_streams = {}


def _side_stream(device) -> "torch.cuda.Stream":
    """A second stream per device (default priority) for the work that can
    run beside the list building."""
    key = torch.device(device).index
    s = _side_streams.get(key)
    if s is None:
        s = torch.cuda.Stream(device=device)
        _side_streams[key] = s
    return s


@dataclass
class StepResult:
    out: torch.Tensor
    lse: Optional[torch.Tensor]
    row_ptr: torch.Tensor
    col: Optional[torch.Tensor]
    lw: Optional[torch.Tensor]
    order: Optional[torch.Tensor]
    perm_q: Optional[torch.Tensor] = None
    perm_k: Optional[torch.Tensor] = None
    crm: Optional[torch.Tensor] = None
    stage1_decision: Optional[torch.Tensor] = None   # device int32 [1] (adaptive skip)
    stage1_stats: Optional[torch.Tensor] = None      # device float64 [7]
    kv_share: bool = False                            # query-head pairs served in one launch
    order2: Optional[torch.Tensor] = None             # second rows of paired launch entries


def _schedule(dw: DeviceWorkload, row_ptr, col, lw, wave_rows: int, n_xcd: int, row_perm, share: bool,
              pairs: bool, stream):
    """Launch tables (order, order2): with ``pairs`` the consecutive query
    blocks of a head with identical lists share an entry (order2 holds the
    second rows), else one row per entry (order2 None)."""
    if pairs:
        return api.schedule_pairs(row_ptr, col, dw.B, dw.Hq, dw.Hkv, dw.nQB, wave_rows, n_xcd, lw=lw,
                                  row_perm=row_perm, stream=stream)
    return api.schedule(row_ptr, dw.B, dw.Hq, dw.Hkv, dw.nQB, wave_rows, n_xcd, stream=stream, row_perm=row_perm,
                        head_step=2 if share else 1, col=col), None


def _stage1_order(dw: DeviceWorkload, row_ptr, col, stage1: str, iters: int, stream):
    """WaveAlign stage 1 in front of the schedule: "off" (no order), "on"
    (the polar spectral order), or "auto" (the adaptive skip decides on the
    device whether the order is computed; when it is not, the order is the
    identity and the schedule equals the "off" one).  Returns (row_perm,
    decision, stats)."""
    if stage1 == "off":
        return None, None, None
    if stage1 not in ("on", "auto"):
        raise ValueError("stage1 must be 'off', 'on' or 'auto'")
    dec = stats = None
    if stage1 == "auto" and not api.spectral_supported(dw.nQB, dw.nQB):
        return None, None, None   # the skip would decide against it: stage 1 cannot run on this shape
    if stage1 == "auto":
        dec, stats = api.stage1_decide(row_ptr, col, dw.B * dw.Hq, dw.nQB, dw.nQB, dw.N, dw.d, dw.block, iters,
                                       stream=stream)
    perm, _ = api.spectral_order(row_ptr, col, dw.B * dw.Hq, dw.nQB, dw.nQB, iters, enable=dec, stream=stream)
    return perm, dec, stats


def kv_share_supported(dw: DeviceWorkload, v_dim_major: bool = True) -> bool:
    """Whether the shape allows the query-head-pair path: an even number of
    query heads per KV head, 128-token blocks, dim-major V."""
    return (dw.Hq // dw.Hkv) % 2 == 0 and dw.block == 128 and v_dim_major


def _kv_share(dw, kv_share, row_ptr, col, lw, v_dim_major, stream) -> bool:
    if kv_share is False:
        return False
    if kv_share not in (True, "auto"):
        raise ValueError("kv_share must be True, False or 'auto'")
    if not kv_share_supported(dw, v_dim_major):
        if kv_share is True:
            raise ValueError("kv_share needs Hq/Hkv even, 128-token blocks and dim-major V")
        return False
    if kv_share is True:
        return True   # the caller vouches for identical rows
    return bool(api.pair_rows_equal(row_ptr, col, dw.B, dw.Hq, dw.Hkv, dw.nQB, lw=lw, stream=stream).item())


def forward(dw: DeviceWorkload, schedule: bool = True, n_xcd: int = 8, wave_rows: int = 0,
            fuse_scatter: bool = True, want_lse: bool = False, attn_events=None,
            v_dim_major: bool = True, stream=None, stage1: str = "auto", stage1_iters: int = 10,
            crm: bool = False, sampler: Optional[dict] = None, fuse_gather: bool = True,
            overlap: bool = False, kv_share="auto", pair_rows: bool = True) -> StepResult:
    """Run every step of the path once.  ``attn_events`` (start, end) are
    recorded around the attention launch on the same stream.  ``stage1``
    selects WaveAlign's stage 1 in front of the schedule: "auto" (the
    adaptive skip decides on the device), "on" or "off"; ``stage1_iters``
    subspace iterations when it runs.  With CRM lists "auto" means "off"
    (the decision reads CSR columns, which CRM rows only give after a host
    round trip).  With ``crm``
    the lists are CRM rows (no log-weights, dim-major V); their sizes are
    known up front, so this path makes no host synchronisation.  With
    ``overlap`` the permutations, gathers and transposes run on a second
    stream while the lists and the schedule are built on this one, and the
    CSR build makes no host round trip (col is sized by its bound).  With
    ``sampler`` = {"m_exact": E, "m_sample": S, "uoff": float64 [B*Hq][G]}
    (a permuted workload) the block mask and log-weights come from the
    group-shared importance sampler over the permuted Q and K instead of
    the workload's mask.  ``kv_share`` (True, False or "auto"): serve the
    identical rows of query-head pairs sharing a KV head in one launch (K/V
    tiles staged once for both heads); "auto" checks the rows on the device
    and uses it where they are identical and the shape allows it.  With
    ``pair_rows`` (and no kv_share, CSR lists, dim-major V, 128-key blocks)
    the schedule pairs consecutive query blocks of a head whose lists are
    identical, and one launch entry serves both rows."""
    crm_rows = None
    if sampler is not None:
        return _forward_sampled(dw, sampler, schedule, n_xcd, wave_rows, fuse_scatter, want_lse, attn_events,
                                stream, stage1, stage1_iters, pair_rows)
    if overlap and not crm:
        return _forward_overlapped(dw, schedule, n_xcd, wave_rows, fuse_scatter, fuse_gather, want_lse,
                                   attn_events, v_dim_major, stream, stage1, stage1_iters, kv_share, pair_rows)
    if crm:
        if dw.lw_map is not None or not v_dim_major:
            raise ValueError("CRM lists carry no log-weights and need dim-major V")
        crm_rows = api.crm_build(dw.mask, dw.T, dw.p, dw.nQB, dw.force_diag, stream=stream)
        row_ptr, _ = api.crm_row_ptr(crm_rows, dw.nQB, want_nnz=False, stream=stream)
        col = lw = None
    else:
        row_ptr, col, lw = api.build_csr(dw.mask, dw.T, dw.p, dw.lw_map, dw.nQB, dw.force_diag,
                                         stream=stream)
    q, k, v = dw.q, dw.k, dw.v
    perm_q = perm_k = None
    if dw.permuted:
        perm_q = api.perm_from_labels(dw.labels_q, dw.n_clusters, stream=stream)
        perm_k = api.perm_from_labels(dw.labels_k, dw.n_clusters, stream=stream)
        if not fuse_gather:
            q = api.permute_rows(dw.q, perm_q, stream=stream)
        k = api.permute_rows(dw.k, perm_k, stream=stream)
        if not v_dim_major:
            v = api.permute_rows(dw.v, perm_k, stream=stream)
    if v_dim_major:
        v = api.transpose_rows(dw.v, perm_k, ld=dw.nQB * dw.block, stream=stream)
    order = dec = stats = row_perm = None
    if schedule:
        if crm and stage1 == "on":
            _, nnz = api.crm_row_ptr(crm_rows, dw.nQB, row_ptr=row_ptr, stream=stream)
            cols = api.crm_to_csr(crm_rows, dw.nQB, row_ptr, nnz, stream=stream)
            row_perm, _, _ = _stage1_order(dw, row_ptr, cols, "on", stage1_iters, stream)
        elif not crm:
            row_perm, dec, stats = _stage1_order(dw, row_ptr, col, stage1, stage1_iters, stream)
    share = False if crm else _kv_share(dw, kv_share, row_ptr, col, lw, v_dim_major, stream)
    order2 = None
    if schedule:
        pairs = pair_rows and not share and not crm and v_dim_major and dw.block == 128
        order, order2 = _schedule(dw, row_ptr, col, lw, wave_rows, n_xcd, row_perm, share, pairs, stream)
    sperm = perm_q if (dw.permuted and fuse_scatter) else None
    s = stream if stream is not None else torch.cuda.current_stream()
    if attn_events is not None:
        attn_events[0].record(s)
    gperm = perm_q if (dw.permuted and fuse_gather) else None
    out, lse = api.attn_fwd(q, k, v, row_ptr, col, dw.block, lw=lw, order=order, scatter_perm_q=sperm,
                            want_lse=want_lse, causal=dw.causal, v_dim_major=v_dim_major, crm=crm_rows,
                            gather_perm_q=gperm, kv_share=share, order2=order2, stream=stream)
    if attn_events is not None:
        attn_events[1].record(s)
    if dw.permuted and not fuse_scatter:
        out = api.unpermute_rows(out, perm_q, stream=stream)
        if lse is not None:
            inv = torch.empty_like(lse)
            inv.scatter_(1, perm_q.long(), lse)
            lse = inv
    return StepResult(out, lse, row_ptr, col, lw, order, perm_q, perm_k, crm_rows, dec, stats, share, order2)


def _forward_sampled(dw: DeviceWorkload, sampler: dict, schedule: bool, n_xcd: int, wave_rows: int,
                     fuse_scatter: bool, want_lse: bool, attn_events, stream, stage1: str,
                     stage1_iters: int, pair_rows: bool = True) -> StepResult:
    """labels -> perms; Q/K gathered, V gathered and transposed; query-group
    and tile centroids; importance-sampled mask and log-weights -> CSR;
    schedule; attention with fused scatter-back."""
    if not dw.permuted:
        raise ValueError("the sampler needs cluster labels")
    perm_q = api.perm_from_labels(dw.labels_q, dw.n_clusters, stream=stream)
    perm_k = api.perm_from_labels(dw.labels_k, dw.n_clusters, stream=stream)
    q = api.permute_rows(dw.q, perm_q, stream=stream)
    k = api.permute_rows(dw.k, perm_k, stream=stream)
    v = api.transpose_rows(dw.v, perm_k, ld=dw.nQB * dw.block, stream=stream)
    q_seg = api.segment_offsets(dw.labels_q, dw.n_clusters, stream=stream)
    qbar = api.segment_means(q, q_seg, stream=stream)
    kbar = api.segment_means(k, seg_len=dw.block, stream=stream)
    mask, lw_map, _ = api.is_sample(qbar, kbar, q_seg, sampler["uoff"], dw.B, dw.Hq, dw.Hkv, dw.N, dw.block,
                                    sampler["m_exact"], sampler["m_sample"], stream=stream)
    row_ptr, col, lw = api.build_csr(mask, None, 0.0, lw_map, dw.nQB, True, stream=stream)
    order = order2 = dec = stats = None
    if schedule:
        row_perm, dec, stats = _stage1_order(dw, row_ptr, col, stage1, stage1_iters, stream)
        order, order2 = _schedule(dw, row_ptr, col, lw, wave_rows, n_xcd, row_perm, False,
                                  pair_rows and dw.block == 128, stream)
    sperm = perm_q if fuse_scatter else None
    s = stream if stream is not None else torch.cuda.current_stream()
    if attn_events is not None:
        attn_events[0].record(s)
    out, lse = api.attn_fwd(q, k, v, row_ptr, col, dw.block, lw=lw, order=order, scatter_perm_q=sperm,
                            want_lse=want_lse, causal=dw.causal, v_dim_major=True, order2=order2, stream=stream)
    if attn_events is not None:
        attn_events[1].record(s)
    if not fuse_scatter:
        out = api.unpermute_rows(out, perm_q, stream=stream)
        if lse is not None:
            inv = torch.empty_like(lse)
            inv.scatter_(1, perm_q.long(), lse)
            lse = inv
    return StepResult(out, lse, row_ptr, col, lw, order, perm_q, perm_k, None, dec, stats, False, order2)


def _forward_overlapped(dw: DeviceWorkload, schedule: bool, n_xcd: int, wave_rows: int, fuse_scatter: bool,
                        fuse_gather: bool, want_lse: bool, attn_events, v_dim_major: bool, stream, stage1: str,
                        stage1_iters: int, kv_share="auto", pair_rows: bool = True) -> StepResult:
    """The same step with two streams: [key labels -> perm_k, K gather, V
    gather + transpose] on a side stream beside [query labels -> perm_q,
    mask -> CSR without a host round trip, schedule] on the caller's stream;
    attention waits for both.  kv_share="auto" reads the pair check's flag
    on the host (the one round trip of this path, taken only on shapes the
    pair kernel serves)."""
    main = stream if stream is not None else torch.cuda.current_stream()
    side = _side_stream(dw.q.device)
    side.wait_stream(main)
    q, k, v = dw.q, dw.k, dw.v
    perm_q = perm_k = None
    with torch.cuda.stream(side):
        if dw.permuted:
            perm_k = api.perm_from_labels(dw.labels_k, dw.n_clusters, stream=side)
            k = api.permute_rows(dw.k, perm_k, stream=side)
            if not v_dim_major:
                v = api.permute_rows(dw.v, perm_k, stream=side)
        if v_dim_major:
            v = api.transpose_rows(dw.v, perm_k, ld=dw.nQB * dw.block, stream=side)
    # the query permutation is only needed by the attention launch (or the
    # explicit Q gather), so it is built here, beside the K/V work
    if dw.permuted:
        perm_q = api.perm_from_labels(dw.labels_q, dw.n_clusters, stream=main)
        if not fuse_gather:
            q = api.permute_rows(dw.q, perm_q, stream=main)
    row_ptr, col, lw = api.build_csr(dw.mask, dw.T, dw.p, dw.lw_map, dw.nQB, dw.force_diag, sync=False,
                                     stream=main)
    order = dec = stats = None
    if schedule:
        row_perm, dec, stats = _stage1_order(dw, row_ptr, col, stage1, stage1_iters, main)
    share = _kv_share(dw, kv_share, row_ptr, col, lw, v_dim_major, main)
    order2 = None
    if schedule:
        pairs = pair_rows and not share and v_dim_major and dw.block == 128
        order, order2 = _schedule(dw, row_ptr, col, lw, wave_rows, n_xcd, row_perm, share, pairs, main)
    main.wait_stream(side)
    for t in (perm_k, k, v):
        if t is not None:
            t.record_stream(main)
    sperm = perm_q if (dw.permuted and fuse_scatter) else None
    gperm = perm_q if (dw.permuted and fuse_gather) else None
    if attn_events is not None:
        attn_events[0].record(main)
    out, lse = api.attn_fwd(q, k, v, row_ptr, col, dw.block, lw=lw, order=order, scatter_perm_q=sperm,
                            want_lse=want_lse, causal=dw.causal, v_dim_major=v_dim_major,
                            gather_perm_q=gperm, kv_share=share, order2=order2, stream=main)
    if attn_events is not None:
        attn_events[1].record(main)
    if dw.permuted and not fuse_scatter:
        out = api.unpermute_rows(out, perm_q, stream=main)
        if lse is not None:
            inv = torch.empty_like(lse)
            inv.scatter_(1, perm_q.long(), lse)
            lse = inv
    return StepResult(out, lse, row_ptr, col, lw, order, perm_q, perm_k, None, dec, stats, share, order2)
