#!/usr/bin/env python3
"""Benchmark: one step = one pass of the whole block-sparse attention path
(threshold map -> CSR beside [cluster labels -> permutations, K gather, V gather
into the dim-major layout] on a second stream, row schedule, attention forward with the query
gather and the scatter-back fused) on a synthetic
Wan2.1-14B-shaped 720p video DiT self-attention (1 x 40 heads x 75600 tokens,
d = 128, 128x128 blocks, 64 Gaussian clusters per head, KV blocks kept to
cumulative mass 0.9, ~15 % density).

Prints one JSON line.  ``value`` is effective TFLOPS of the whole step
(4*d FLOPs per allowed query-key pair / step time); ``roofline`` is measured
on the attention kernel alone with HIP events on its stream; ``cpu_baseline``
times the CPU reference checker on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn fwd effective TFLOPS & % bf16 MFMA peak, Wan2.1-14B shape"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="clustered",
                    choices=["clustered", "importance_sampled", "video_threshold", "llm_prefill", "tiny"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU-baseline work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-token-sets", action="store_true", help="skip the token-level set measurements")
    ap.add_argument("--no-selection", action="store_true", help="skip the exact-selection (anchor step) measurements")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip every measurement beside the headline step (CRM lists, sampler, token sets), "
                         "so that a profile holds only the headline kernel's launches")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for HBM counter scaling)")
    ap.add_argument("--dense-launches", type=int, default=0,
                    help="instead of the step: launch the attention kernel this many times on dense "
                         "1x40x16384 heads (every 128x128 block listed), print the median, and exit "
                         "(a short, fixed program for counter passes)")
    ap.add_argument("--selection-only", action="store_true",
                    help="instead of the step: run only the exact-selection (anchor step) measurements, "
                         "print them as one JSON line, and exit")
    ap.add_argument("--token-sets-only", action="store_true",
                    help="instead of the step: run only the token-level set measurements and print them")
    ap.add_argument("--pair-rows-ab", default="",
                    help="instead of the step: time the attention of the named workloads (comma-separated) "
                         "with one row per launch entry and with identical consecutive rows paired, alternating, "
                         "print one JSON line and exit")
    ap.add_argument("--kv-share-ab", action="store_true",
                    help="instead of the step: time the LLaMA-3.1-8B prefill workload's attention alone with "
                         "the per-head kernel and with the query-head-pair kernel (alternating, median of 20 "
                         "each), compare their outputs, print one JSON line and exit")
    ap.add_argument("--n-xcd", type=int, default=8)
    ap.add_argument("--wave-rows", type=int, default=0)
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the kernel lines of the Wan2.1-1.3B threshold, importance-sampled and "
                         "LLaMA-3.1-8B prefill workloads")
    ap.add_argument("--summarize-profile", metavar="DIR", default=None,
                    help="instead of the step: read the kernel trace and the FETCH_SIZE / WRITE_SIZE / TCC "
                         "counter runs of the headline kernel under DIR (rocprofv3 csv output: "
                         "DIR/{trace,fetch,write,tcc}) and write profiles/attn_wan14b_clustered_traffic.json")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def dense_launches(torch, n):
    """Dense 1 x 40 x 16384 heads, d = 128, every 128x128 block listed, V
    dim-major, longest-first schedule: n launches of the attention kernel,
    each timed with HIP events on the current stream; prints the median."""
    from block_sparse_attention_mask_amd import api
    H, N = 40, 16384
    g = torch.Generator(device="cuda").manual_seed(0)
    q, k, v = (torch.randn(1, H, N, 128, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    vt = api.transpose_rows(v)
    nb = N // 128
    rp, col, _ = api.build_csr(torch.ones(H * nb, nb, dtype=torch.uint8, device="cuda"), nQB=nb)
    order = api.schedule(rp, 1, H, H, nb, 0, 8, col=col)
    out = torch.empty_like(q)
    s = torch.cuda.current_stream()
    ms = []
    for _ in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        api.attn_fwd(q, k, vt, rp, col, 128, order=order, out=out, v_dim_major=True)
        b.record(s)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    t = float(np.median(ms))
    flop = 4.0 * 128 * H * N * N
    print(json.dumps({"workload": "dense 1x40x16384, d128, 128x128 blocks", "launches": n, "median_ms": round(t, 4),
                      "tflops": round(flop / (t * 1e-3) / 1e12, 2)}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    import torch

    from block_sparse_attention_mask_amd import _lib, metrics, pipeline
    import synth
    if not os.path.exists(_lib.LIB_PATH):
        raise SystemExit("libbsattn.so is not built; run python __graft_entry__.py first")
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.dense_launches:
        dense_launches(torch, args.dense_launches)
        return
    if args.selection_only:
        print(json.dumps({"exact_selection": selection_stage(torch)}), flush=True)
        return
    if args.token_sets_only:
        print(json.dumps({"token_sets": token_set_stage(torch)}), flush=True)
        return
    if args.kv_share_ab:
        print(json.dumps({"kv_share_ab": kv_share_ab(args, torch)}), flush=True)
        return
    if args.pair_rows_ab:
        print(json.dumps({"pair_rows_ab": pair_rows_ab(args, torch)}), flush=True)
        return

    t0 = time.time()
    w = synth.CONFIGS[args.config]()
    log("generated %s in %.1fs" % (args.config, time.time() - t0))
    dw = pipeline.to_device(w, dev)
    stream = torch.cuda.current_stream()

    # one pass to get the CSR for the work count (outside the timed region);
    # it also writes the LSE the oracle leg checks
    res = pipeline.forward(dw, n_xcd=args.n_xcd, wave_rows=args.wave_rows, overlap=True, want_lse=True)
    torch.cuda.synchronize()
    head_kernel = attn_kernel_name(w.block, w.d, res.kv_share, res.order2 is not None)
    rp = res.row_ptr.cpu().numpy()
    col = res.col[:int(rp[-1])].cpu().numpy()   # col is sized by its bound
    stage1 = stage1_record(res)
    pairs = metrics.count_pairs(rp, col, w.N, w.block, w.causal)
    eff_flops = 4.0 * w.d * pairs
    nnz = int(rp[-1])
    density = nnz / float(w.R * w.nKB)
    log("nnz %d density %.4f pairs %d eff GFLOP %.1f" % (nnz, density, pairs, eff_flops / 1e9))

    for _ in range(args.warmup):
        pipeline.forward(dw, n_xcd=args.n_xcd, wave_rows=args.wave_rows, overlap=True)
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    last = None
    for i in range(args.steps):
        last = pipeline.forward(dw, n_xcd=args.n_xcd, wave_rows=args.wave_rows, overlap=True, attn_events=evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = t_total * 1e3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg = float(np.mean(attn_ms))
    attn_med = float(np.median(attn_ms))
    value = eff_flops / (ms_step * 1e-3) / 1e12
    attn_tflops = eff_flops / (attn_avg * 1e-3) / 1e12
    log("step %.3f ms, attention avg %.3f ms (median %.3f) -> %.1f TFLOPS kernel, %.1f TFLOPS step"
        % (ms_step, attn_avg, attn_med, attn_tflops, value))

    # stage breakdown (one extra, separately synchronised pass; not part of value)
    stages = stage_times(pipeline, dw, args, torch)
    # the attention launch alone: 10 warm-up calls, median of 50; then one
    # launch after a 1 GiB write has evicted L2 and MALL
    attn_solo = attention_alone(dw, args, torch)
    # the same launch with CRM rows in place of the CSR lists (workloads
    # without log-weights), and the mask -> CRM stage
    crm = None
    if dw.lw_map is None and not args.headline_only:
        crm_solo = attention_alone(dw, args, torch, crm=True)
        W = -(-w.nQB // 32)
        crm = {"alone_median50_ms": crm_solo["median_ms"], "l2_flushed_ms": crm_solo["flushed_ms"],
               "mask_to_crm_ms": crm_stage_ms(dw, torch),
               "list_bytes_per_row": {"crm": 4 * W, "csr": round(4.0 + 4.0 * nnz / w.R, 1)}}

    # the device importance sampler (8 exact + 8 sampled tiles per query
    # group) on the same permuted Q and K, and attention on its lists
    sampled = sampler_stage(dw, torch) if (dw.permuted and not args.headline_only) else None

    # token-level computational query sets (INTRA Scatter / Gather 0,
    # MC-Sparse-shaped token selection) on their own synthetic inputs
    token_sets = None if (args.no_token_sets or args.headline_only) else token_set_stage(torch)
    # MC-Sparse's anchor step: dense pass, exact selection, sparse attention
    selection = None if (args.no_selection or args.headline_only) else selection_stage(torch)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: %d MiB x3 (torch copy kernel)" % args.copy_probe_mib)

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on the row set of the measurement protocol, against the
        # output of the last timed step (O) and of the work-count pass (LSE)
        cpu = oracle_leg(w, last.out, res.lse, (rp, col), torch)
        log("oracle leg: %s" % {k: v for k, v in cpu.items() if k != "sample"})

    # the other page-shaped workloads: kernel alone, error on the sampled
    # rows, oracle timing
    others = None
    if not (args.no_other_workloads or args.headline_only):
        del dw, res, last
        torch.cuda.empty_cache()
        others = {}
        for cfg in ("video_threshold", "importance_sampled", "llm_prefill"):
            others[cfg] = workload_line(cfg, args, torch, with_oracle=not args.no_cpu_baseline)
            torch.cuda.empty_cache()

    dev = device_info(torch)
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload_name(args.config),
            "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "seq_len": w.N, "head_dim": w.d,
            "block": w.block, "nnz_blocks": nnz, "block_density": round(density, 5),
            "allowed_pairs": pairs, "effective_gflop": round(eff_flops / 1e9, 3),
            "permuted": bool(w.permuted), "causal": bool(w.causal), "log_weights": w.lw_map is not None,
            "schedule": {"n_xcd": args.n_xcd, "wave_rows": args.wave_rows or "auto"},
            "parallelism": "single-gpu",
        },
        "pct_bf16_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "attn_kernel": {"avg_ms": round(attn_avg, 4), "median_ms": round(attn_med, 4),
                        "tflops": round(attn_tflops, 2),
                        "pct_bf16_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
                        "alone_median50_ms": attn_solo["median_ms"],
                        "alone_median50_tflops": round(eff_flops / (attn_solo["median_ms"] * 1e-3) / 1e12, 2),
                        "l2_flushed_ms": attn_solo["flushed_ms"]},
        "device": dev,
        "stages_ms": stages,
        "stage1_adaptive_skip": stage1,
        "crm_lists": crm,
        "importance_sampler": sampled,
        "token_sets": token_sets,
        "exact_selection": selection,
        "roofline": dict({"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4)},
                         **profile_record(args.config),
                         **{"traffic_unit": "HBM-side bytes per launch (scaled FETCH_SIZE + WRITE_SIZE)",
                            "frac_of_mfma_rate_random_bf16": round(
                                attn_tflops / dev["mfma_random_bf16_operands"]["tflops"], 4),
                            "kernel": head_kernel,
                            "per_unit": "4*d = 512 FLOP per allowed query-key pair",
                            "units_per_launch": pairs}),
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(out), flush=True)
    bad = [(n, c) for n, c in [("headline", cpu)] + list((others or {}).items())
           if c and not c.get("within_tolerance", True)]
    if bad:
        log("OUTPUT OUTSIDE THE TOLERANCE (max-abs 2e-2, mean-abs 2e-3) ON: %s" % [n for n, _ in bad])
        sys.exit(3)


def attn_kernel_name(block, d, kv_share=False, pairs=False):
    """The attention kernel bsa_attn_fwd launches for dim-major V."""
    if kv_share:
        return "attn_ppg_128_%d" % d
    if pairs and block == 128:
        return "attn_ppx_128_%d" % d
    return ("attn_pp_128_%d" % d) if block == 128 else ("attn_dimv_%d_%d" % (block, d))


ATTN_SOURCES = ("attn_pp.hip", "attn_pp_body.h", "attn_ppg.hip", "attn_dimv.hip", "attn_common.h", "attn_fwd.hip",
                "bsa_internal.h", "schedule.hip")


def attn_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, "block_sparse_attention_mask_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def kv_share_ok(dw, row_ptr, col, lw):
    """Whether the query-head-pair kernel serves this workload: the shape
    allows it and the pair check finds the rows identical."""
    from block_sparse_attention_mask_amd import api, pipeline
    if col is None or not pipeline.kv_share_supported(dw):
        return False
    return bool(api.pair_rows_equal(row_ptr, col, dw.B, dw.Hq, dw.Hkv, dw.nQB, lw=lw).item())


def attention_alone(dw, args, torch, crm=False):
    """The attention kernel by itself on its inputs (already permuted and
    transposed), timed with HIP events on the current stream.  With ``crm``
    the lists are CRM rows."""
    from block_sparse_attention_mask_amd import api
    crm_rows = None
    if crm:
        crm_rows = api.crm_build(dw.mask, dw.T, dw.p, dw.nQB, dw.force_diag)
        row_ptr, _ = api.crm_row_ptr(crm_rows, dw.nQB, want_nnz=False)
        col = lw = None
    else:
        row_ptr, col, lw = api.build_csr(dw.mask, dw.T, dw.p, dw.lw_map, dw.nQB, dw.force_diag)
    q, k, pq, pk = dw.q, dw.k, None, None
    if dw.permuted:
        pq = api.perm_from_labels(dw.labels_q, dw.n_clusters)
        pk = api.perm_from_labels(dw.labels_k, dw.n_clusters)
        k = api.permute_rows(dw.k, pk)
    v = api.transpose_rows(dw.v, pk, ld=dw.nQB * dw.block)
    share = kv_share_ok(dw, row_ptr, col, lw) and not crm
    order2 = None
    if not share and not crm and dw.block == 128:   # identical consecutive rows paired, as in the step
        order, order2 = api.schedule_pairs(row_ptr, col, dw.B, dw.Hq, dw.Hkv, dw.nQB, args.wave_rows, args.n_xcd,
                                           lw=lw)
    else:
        order = api.schedule(row_ptr, dw.B, dw.Hq, dw.Hkv, dw.nQB, args.wave_rows, args.n_xcd,
                             head_step=2 if share else 1, col=col)
    out = torch.empty((dw.B, dw.Hq, dw.N, dw.d), dtype=q.dtype, device=q.device)

    def launch():   # the query gather and the output scatter are fused into the kernel
        api.attn_fwd(q, k, v, row_ptr, col, dw.block, lw=lw, order=order, scatter_perm_q=pq,
                     gather_perm_q=pq, causal=dw.causal, v_dim_major=True, out=out, crm=crm_rows,
                     kv_share=share, order2=order2)

    for _ in range(10):
        launch()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
    for a, b in ev:
        a.record(s)
        launch()
        b.record(s)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    flush = torch.empty(1 << 29, dtype=torch.int16, device=q.device)
    flush.fill_(1)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    launch()
    b.record(s)
    torch.cuda.synchronize()
    del flush
    return {"median_ms": round(float(np.median(ms)), 4), "flushed_ms": round(a.elapsed_time(b), 4)}


def crm_stage_ms(dw, torch):
    """Mask -> CRM rows and their row offsets (no host synchronisation):
    median of 10 after 2 warm-up passes."""
    from block_sparse_attention_mask_amd import api
    s = torch.cuda.current_stream()
    crm = api.crm_build(dw.mask, dw.T, dw.p, dw.nQB, dw.force_diag)
    rp, _ = api.crm_row_ptr(crm, dw.nQB, want_nnz=False)
    ms = []
    for i in range(12):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        api.crm_build(dw.mask, dw.T, dw.p, dw.nQB, dw.force_diag, crm=crm)
        api.crm_row_ptr(crm, dw.nQB, row_ptr=rp, want_nnz=False)
        b.record(s)
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(a.elapsed_time(b))
    return round(float(np.median(ms)), 4)


def sampler_stage(dw, torch, m_exact=8, m_sample=8):
    """Median of 10 (after 2 warm-up passes) of each step of the sampled
    mask: query-group offsets, query-group and tile centroids, the sampler,
    the CSR build; then the attention launch on the sampled lists."""
    from block_sparse_attention_mask_amd import api
    s = torch.cuda.current_stream()
    pq = api.perm_from_labels(dw.labels_q, dw.n_clusters)
    pk = api.perm_from_labels(dw.labels_k, dw.n_clusters)
    q = api.permute_rows(dw.q, pq)
    k = api.permute_rows(dw.k, pk)
    v = api.transpose_rows(dw.v, pk, ld=dw.nQB * dw.block)
    gen = torch.Generator(device="cpu").manual_seed(4321)
    uoff = torch.rand((dw.B * dw.Hq, dw.n_clusters), generator=gen, dtype=torch.float64).to(q.device)
    names = ["segment_offsets", "query_centroids", "tile_centroids", "is_sample", "mask_to_csr"]
    times = {n: [] for n in names}
    res = None
    for it in range(12):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record(s)
        seg = api.segment_offsets(dw.labels_q, dw.n_clusters)
        ev[1].record(s)
        qbar = api.segment_means(q, seg)
        ev[2].record(s)
        kbar = api.segment_means(k, seg_len=dw.block)
        ev[3].record(s)
        mask, lw_map, _ = api.is_sample(qbar, kbar, seg, uoff, dw.B, dw.Hq, dw.Hkv, dw.N, dw.block, m_exact,
                                        m_sample)
        ev[4].record(s)
        res = api.build_csr(mask, None, 0.0, lw_map, dw.nQB, True)
        ev[5].record(s)
        torch.cuda.synchronize()
        if it >= 2:
            for i, n in enumerate(names):
                times[n].append(ev[i].elapsed_time(ev[i + 1]))
    row_ptr, col, lw = res
    order = api.schedule(row_ptr, dw.B, dw.Hq, dw.Hkv, dw.nQB, 0, 8, col=col)
    ms = []
    for it in range(12):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        api.attn_fwd(q, k, v, row_ptr, col, dw.block, lw=lw, order=order, scatter_perm_q=pq, v_dim_major=True)
        b.record(s)
        torch.cuda.synchronize()
        if it >= 2:
            ms.append(a.elapsed_time(b))
    from block_sparse_attention_mask_amd import metrics
    nnz = int(row_ptr[-1].item())
    pairs = metrics.count_pairs(row_ptr.cpu().numpy(), col[:nnz].cpu().numpy(), dw.N, dw.block, dw.causal)
    att = float(np.median(ms))
    out = {n: round(float(np.median(t)), 4) for n, t in times.items()}
    out.update({"budget_tiles": {"exact": m_exact, "sampled": m_sample}, "nnz_blocks": nnz,
                "attention_ms": round(att, 4),
                "attention_tflops": round(4.0 * dw.d * pairs / (att * 1e-3) / 1e12, 2)})
    return out


def kv_share_ab(args, torch):
    """The LLaMA-3.1-8B prefill workload's attention alone, per-head kernel
    (one row per workgroup) against the query-head-pair kernel (one
    workgroup per pair of identical rows of query heads 2j, 2j + 1): both
    launched on the same inputs, alternating, 10 warm-up calls and 20 timed
    launches each; the two outputs are compared (the same function up to
    rounding order)."""
    from block_sparse_attention_mask_amd import api, metrics, pipeline
    import synth
    w = synth.CONFIGS["llm_prefill"]()
    dw = pipeline.to_device(w, torch.device("cuda"))
    row_ptr, col, lw = api.build_csr(dw.mask, dw.T, dw.p, dw.lw_map, dw.nQB, dw.force_diag)
    if not kv_share_ok(dw, row_ptr, col, lw):
        raise SystemExit("the prefill rows are not pair-identical")
    v = api.transpose_rows(dw.v, None, ld=dw.nQB * dw.block)
    outs, launches = {}, {}
    for share in (False, True):
        order = api.schedule(row_ptr, dw.B, dw.Hq, dw.Hkv, dw.nQB, args.wave_rows, args.n_xcd,
                             head_step=2 if share else 1, col=col)
        out = torch.empty((dw.B, dw.Hq, dw.N, dw.d), dtype=dw.q.dtype, device=dw.q.device)
        outs[share] = out
        launches[share] = (lambda o=order, out=out, share=share: api.attn_fwd(
            dw.q, dw.k, v, row_ptr, col, dw.block, lw=lw, order=o, causal=dw.causal, v_dim_major=True,
            out=out, kv_share=share))
    s = torch.cuda.current_stream()
    for _ in range(10):
        for share in (False, True):
            launches[share]()
    ms = {False: [], True: []}
    for _ in range(20):
        for share in (False, True):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            launches[share]()
            b.record(s)
            torch.cuda.synchronize()
            ms[share].append(a.elapsed_time(b))
    rp = row_ptr.cpu().numpy()
    nnz = int(rp[-1])
    pairs = metrics.count_pairs(rp, col[:nnz].cpu().numpy(), w.N, w.block, w.causal)
    flop = 4.0 * w.d * pairs
    as_f32 = lambda t: (t.view(torch.bfloat16) if t.dtype in (torch.int16, torch.uint16) else t).float()
    diff = (as_f32(outs[False]) - as_f32(outs[True])).abs()
    res = {"workload": workload_name("llm_prefill"), "effective_gflop": round(flop / 1e9, 3),
           "max_abs_diff": float(diff.max().item()), "mean_abs_diff": float(diff.mean().item())}
    for share, key in ((False, "per_head"), (True, "head_pairs")):
        t = float(np.median(ms[share]))
        res[key] = {"kernel": attn_kernel_name(w.block, w.d, share), "median_ms": round(t, 4),
                    "tflops": round(flop / (t * 1e-3) / 1e12, 2),
                    "frac": round(flop / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    log("kv_share A/B: per head %.3f ms, head pairs %.3f ms" % (res["per_head"]["median_ms"],
                                                                res["head_pairs"]["median_ms"]))
    return res


def pair_rows_ab(args, torch):
    """Attention alone (query gather and output scatter fused) on each named
    workload with one row per launch entry (bsa_schedule, attn_pp) and with
    identical consecutive rows paired (bsa_schedule_pairs, attn_ppx): both on
    the same inputs, alternating, 10 warm-up rounds and 20 timed launches
    each; the outputs are compared (the same function up to rounding
    order)."""
    from block_sparse_attention_mask_amd import api, metrics, pipeline
    import synth
    res = {}
    for cfg in args.pair_rows_ab.split(","):
        w = synth.CONFIGS[cfg]()
        dw = pipeline.to_device(w, torch.device("cuda"))
        row_ptr, col, lw = api.build_csr(dw.mask, dw.T, dw.p, dw.lw_map, dw.nQB, dw.force_diag)
        q, k, pq, pk = dw.q, dw.k, None, None
        if dw.permuted:
            pq = api.perm_from_labels(dw.labels_q, dw.n_clusters)
            pk = api.perm_from_labels(dw.labels_k, dw.n_clusters)
            k = api.permute_rows(dw.k, pk)
        v = api.transpose_rows(dw.v, pk, ld=dw.nQB * dw.block)
        tables = {"rows": (api.schedule(row_ptr, dw.B, dw.Hq, dw.Hkv, dw.nQB, args.wave_rows, args.n_xcd, col=col),
                           None),
                  "pairs": api.schedule_pairs(row_ptr, col, dw.B, dw.Hq, dw.Hkv, dw.nQB, args.wave_rows, args.n_xcd,
                                              lw=lw)}
        outs, launches = {}, {}
        for key, (o, o2) in tables.items():
            out = torch.empty((dw.B, dw.Hq, dw.N, dw.d), dtype=q.dtype, device=q.device)
            outs[key] = out
            launches[key] = (lambda o=o, o2=o2, out=out: api.attn_fwd(
                q, k, v, row_ptr, col, dw.block, lw=lw, order=o, order2=o2, scatter_perm_q=pq, gather_perm_q=pq,
                causal=dw.causal, v_dim_major=True, out=out))
        s = torch.cuda.current_stream()
        for _ in range(10):
            for key in launches:
                launches[key]()
        ms = {key: [] for key in launches}
        for _ in range(20):
            for key in launches:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(s)
                launches[key]()
                b.record(s)
                torch.cuda.synchronize()
                ms[key].append(a.elapsed_time(b))
        rp = row_ptr.cpu().numpy()
        nnz = int(rp[-1])
        pairs = metrics.count_pairs(rp, col[:nnz].cpu().numpy(), w.N, w.block, w.causal)
        flop = 4.0 * w.d * pairs
        as_f32 = lambda t: (t.view(torch.bfloat16) if t.dtype in (torch.int16, torch.uint16) else t).float()
        diff = (as_f32(outs["rows"]) - as_f32(outs["pairs"])).abs()
        r = {"workload": workload_name(cfg), "launch_entries": int(rp.size - 1),
             "pair_entries": int((tables["pairs"][1] >= 0).sum().item()),
             "max_abs_diff": float(diff.max().item()), "mean_abs_diff": float(diff.mean().item())}
        for key, kern in (("rows", attn_kernel_name(w.block, w.d)), ("pairs", attn_kernel_name(w.block, w.d, pairs=True))):
            t = float(np.median(ms[key]))
            r[key] = {"kernel": kern, "median_ms": round(t, 4), "tflops": round(flop / (t * 1e-3) / 1e12, 2),
                      "frac": round(flop / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log("%s: one row per entry %.3f ms, pairs %.3f ms (%d pair entries)" % (
            cfg, r["rows"]["median_ms"], r["pairs"]["median_ms"], r["pair_entries"]))
        res[cfg] = r
        del dw, outs, launches, q, k, v
        torch.cuda.empty_cache()
    return res


def token_set_stage(torch):
    """Token-level attention over computational query sets: median of 10
    launches after 3 warm-up calls, effective TFLOPS (4 d per allowed pair).
    Q, K, V ~ N(0, 1) in bf16 from a seeded device generator."""
    from block_sparse_attention_mask_amd import api
    import synth
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(2024)
    res = {}

    def qkv(Hq, Hkv, N, d=128):
        f = lambda H: torch.randn((1, H, N, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        return f(Hq), f(Hkv), f(Hkv)

    def timed(name, shape, q, k, v, q_idx, kv_ptr, kv_idx, causal, pairs, kv_share=False):
        out = torch.empty_like(q)
        for _ in range(3):
            api.attn_tok_fwd(q, k, v, q_idx, kv_ptr, kv_idx, out=out, causal=causal, kv_share=kv_share)
        s = torch.cuda.current_stream()
        ms = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            api.attn_tok_fwd(q, k, v, q_idx, kv_ptr, kv_idx, out=out, causal=causal, kv_share=kv_share)
            b.record(s)
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        t = float(np.median(ms))
        tf = 4.0 * q.shape[3] * pairs / (t * 1e-3) / 1e12
        res[name] = {"shape": shape, "ms": round(t, 4), "tflops": round(tf, 2),
                     "pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "allowed_pairs": int(pairs)}
        log("token sets %s: %.3f ms, %.1f TFLOPS" % (name, t, tf))

    # INTRA Scatter, LLaMA-3.1-8B prefill shape at 32K: 8 relay groups, causal
    N, Hq, Hkv, R = 32768, 32, 8, 8
    maps = synth.cqs_per_head(synth.cqs_scatter(N, R, 64, True), Hq)
    T = N // R
    pairs = Hq * R * T * (T + 1) // 2
    qkv_s = qkv(Hq, Hkv, N)
    timed("intra_scatter_llama3_8b_32k", "1x32q/8kv x 32768, d128, 8 groups, causal, 64-query sets",
          *qkv_s, *(torch.from_numpy(x).to(dev) for x in maps), True, pairs)
    # the same sets served per pair of query heads of a KV group (the map is
    # the same for every head): each gathered K/V tile serves both heads
    timed("intra_scatter_llama3_8b_32k_head_pairs", "same, one workgroup per pair of query heads sharing a KV head",
          *qkv_s, *(torch.from_numpy(x).to(dev) for x in maps), True, pairs, kv_share=True)
    # ... and per run of the four query heads of a KV head (GQA-4)
    timed("intra_scatter_llama3_8b_32k_head_quads", "same, one workgroup per four query heads sharing a KV head",
          *qkv_s, *(torch.from_numpy(x).to(dev) for x in maps), True, pairs, kv_share=4)
    # the same pattern executed as 128-query sets (two consecutive 64-query
    # sets of a group share the later one's key list; causal masking keeps
    # the computation identical)
    maps = synth.cqs_per_head(synth.cqs_scatter(N, R, 128, True), Hq)
    timed("intra_scatter_llama3_8b_32k_sets128", "same, 128-query sets",
          *qkv_s, *(torch.from_numpy(x).to(dev) for x in maps), True, pairs)
    # INTRA Gather 1 on the same shape: segments of 8 tokens dealt cyclically to 8 groups, causal
    maps = synth.cqs_per_head(synth.cqs_gather1(N, R, 64, True), Hq)
    timed("intra_gather1_llama3_8b_32k", "1x32q/8kv x 32768, d128, 8 groups of cyclic 8-token segments, causal, "
          "64-query sets", *qkv_s, *(torch.from_numpy(x).to(dev) for x in maps), True, pairs)
    timed("intra_gather1_llama3_8b_32k_head_pairs", "same, one workgroup per pair of query heads sharing a KV head",
          *qkv_s, *(torch.from_numpy(x).to(dev) for x in maps), True, pairs, kv_share=True)
    timed("intra_gather1_llama3_8b_32k_head_quads", "same, one workgroup per four query heads sharing a KV head",
          *qkv_s, *(torch.from_numpy(x).to(dev) for x in maps), True, pairs, kv_share=4)
    del qkv_s
    # INTRA Gather 0, FLUX.1-dev 2048x2048 image (128x128 tokens): 8x8 patches, 16x16 windows
    H = W = 128
    heads = 24
    maps = synth.cqs_per_head(synth.cqs_gather0(H, W), heads)
    timed("intra_gather0_flux_128x128", "1x24 x 16384 image tokens, d128, 8x8 query patches, 16x16 key windows",
          *qkv(heads, heads, H * W), *(torch.from_numpy(x).to(dev) for x in maps), False, heads * H * W * 256)
    # token-level KV selection, Wan2.1-14B shape: 128-query groups, 15 % of the keys each
    N, heads, BQ = 75600, 40, 128
    K = int(0.15 * N)
    C = -(-N // BQ)
    q_idx = torch.arange(C * BQ, device=dev, dtype=torch.int32).reshape(1, C, BQ)
    q_idx = torch.where(q_idx < N, q_idx, torch.full_like(q_idx, -1)).expand(heads, C, BQ).contiguous()
    parts = []
    for h in range(heads):
        r = torch.rand((C, N), generator=gen, device=dev)
        parts.append(torch.topk(r, K, dim=1).indices.sort(dim=1).values.to(torch.int32).reshape(-1))
        del r
    kv_idx = torch.cat(parts)
    del parts
    kv_ptr = (torch.arange(heads * C + 1, device=dev, dtype=torch.int64) * K).to(torch.int32)
    timed("token_select_wan14b_15pct", "1x40 x 75600, d128, 128-query groups, 11340 keys each",
          *qkv(heads, heads, N), q_idx, kv_ptr, kv_idx, False, heads * N * K)
    del kv_idx
    torch.cuda.empty_cache()
    return res


def selection_stage(torch):
    """MC-Sparse's anchor step (Algorithm 1) at Wan2.1-14B 720p: V to the
    dim-major layout, the dense pass with log-sum-exp, exact selection (group mass, then top-K at 15 %
    density) and token-level sparse attention on the selected keys; median of
    5 launches of each after 2 warm-up rounds.  Groups are 128 consecutive
    tokens of the (grouped) sequence; Q, K, V ~ N(0, 1) in bf16."""
    from block_sparse_attention_mask_amd import api
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(2025)
    N, H, BQ, d = 75600, 40, 128, 128
    K = int(0.15 * N)
    C = -(-N // BQ)
    f = lambda: torch.randn((1, H, N, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q, k, v = f(), f(), f()
    q_idx = torch.arange(C * BQ, device=dev, dtype=torch.int32).reshape(1, C, BQ)
    q_idx = torch.where(q_idx < N, q_idx, torch.full_like(q_idx, -1)).expand(H, C, BQ).contiguous()
    nQB = -(-N // 128)
    mask = torch.ones((H * nQB, nQB), dtype=torch.uint8, device=dev)
    row_ptr, col, _ = api.build_csr(mask=mask, nQB=nQB)
    del mask
    o_full = torch.empty_like(q)
    vt = api.transpose_rows(v)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)
    mass = torch.empty((H * C, N), dtype=torch.float32, device=dev)
    sel = torch.empty((H * C, K), dtype=torch.int32, device=dev)
    kv_ptr = (torch.arange(H * C + 1, device=dev, dtype=torch.int64) * K).to(torch.int32)
    o_sparse = torch.zeros_like(q)
    steps = {
        "v_transpose": lambda: api.transpose_rows(v, dst=vt),
        "dense_lse": lambda: api.attn_fwd(q, k, vt, row_ptr, col, 128, out=o_full, lse=lse, v_dim_major=True),
        "group_mass": lambda: api.group_mass(q, k, lse, q_idx, out=mass),
        "topk": lambda: api.topk_rows(mass, K, out=sel),
        "sparse_attn": lambda: api.attn_tok_fwd(q, k, v, q_idx, kv_ptr, sel.view(-1), out=o_sparse),
    }
    for _ in range(2):
        for fn in steps.values():
            fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ms = {}
    for name, fn in steps.items():
        t = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(s)
            fn()
            b.record(s)
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        ms[name] = float(np.median(t))
    pairs = H * N * N
    res = {
        "shape": "1x40 x 75600, d128, 128-query groups, K = 11340 (15 %)",
        "ms": {n_: round(t, 4) for n_, t in ms.items()},
        "anchor_ms": round(sum(ms.values()), 4),
        "dense_tflops": round(4.0 * d * pairs / (ms["dense_lse"] * 1e-3) / 1e12, 2),
        "mass_tflops": round(2.0 * d * pairs / (ms["group_mass"] * 1e-3) / 1e12, 2),
        "mass_flop_note": "2*d FLOP per (query, key) pair: the score product; one exp per pair on top",
        "topk_gbps": round(H * C * N * 4 / (ms["topk"] * 1e-3) / 1e9, 1),
        "sparse_tflops": round(4.0 * d * H * N * K / (ms["sparse_attn"] * 1e-3) / 1e12, 2),
    }
    log("exact selection: %s" % res)
    del q, k, v, vt, o_full, lse, mass, sel, o_sparse, row_ptr, col
    torch.cuda.empty_cache()
    return res


def device_info(torch):
    from block_sparse_attention_mask_amd import api
    p = torch.cuda.get_device_properties(0)
    # the matrix cores with constant operands, then with random bf16 operands
    # (every MFMA sees new bits, as on the workloads' inputs): the engine
    # clock, and so the rate, falls with the operand bits that switch.  A
    # short call of each kind first, so that neither reads a cold start.
    api.clock_under_mfma_load(iters=4000)
    api.clock_under_mfma_load(iters=4000, random_operands=True)
    return {"name": p.name, "arch": p.gcnArchName, "cus": api.device_cus(),
            "peak_sclk_mhz": api.device_clock_khz() // 1000,
            "sclk_mhz_under_mfma_load": api.clock_under_mfma_load(),
            "mfma_random_bf16_operands": api.clock_under_mfma_load(random_operands=True)}


def profile_record(cfg):
    """traffic (bytes per launch), L2 hit rate, achieved HBM GB/s and the
    kernel-trace average from the committed counter summary of the headline
    kernel, or nulls when that summary is for another workload or for other
    kernel sources."""
    nulls = {"traffic": None, "l2_hit_rate": None, "hbm_gbs": None, "profile_trace_avg_ms": None}
    if cfg != "clustered":
        return nulls
    path = os.path.join(ROOT, "profiles", "attn_wan14b_clustered_traffic.json")
    if not os.path.exists(path):
        return nulls
    rec = json.load(open(path))
    if attn_sources_sha256() != rec.get("kernel_sources_sha256"):
        return nulls
    return {"traffic": int(rec["traffic_bytes_per_launch"]), "l2_hit_rate": rec["l2_hit_rate"],
            "hbm_gbs": rec["achieved_hbm_gbs"], "profile_trace_avg_ms": rec["trace_avg_ms"]}


def summarize_profile(d):
    """Write profiles/attn_wan14b_clustered_traffic.json from rocprofv3 csv
    output under d: trace/ (--kernel-trace), fetch/ (--pmc FETCH_SIZE), write/
    (--pmc WRITE_SIZE) and tcc/ (--pmc TCC_HIT_sum TCC_MISS_sum), each from
    `bench.py --steps 1 --warmup 0 --no-cpu-baseline --headline-only`, the
    fetch and write runs with `--copy-probe-mib 1024`.  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are scaled by what they read for the
    1 GiB device copy of the same run."""
    import csv
    import glob
    import statistics
    ksub = "attn_ppx_128_128("

    def rows(sub, suffix):
        f = glob.glob(os.path.join(d, sub, "*" + suffix))
        if not f:
            raise SystemExit("no %s under %s" % (suffix, os.path.join(d, sub)))
        return list(csv.DictReader(open(f[0])))

    def counter(sub, name):
        per, names = {}, {}
        for r in rows(sub, "counter_collection.csv"):
            k = int(r["Dispatch_Id"])
            per[k] = per.get(k, 0.0) + float(r["Counter_Value"]) if r["Counter_Name"] == name else per.get(k, 0.0)
            names[k] = r["Kernel_Name"]
        attn = [per[k] for k in sorted(per) if ksub in names[k]]
        copies = [per[k] for k in sorted(per) if "copy" in names[k].lower() and ksub not in names[k]]
        return attn, copies

    probe_kib = 1024.0 * 1024.0
    f, fc = counter("fetch", "FETCH_SIZE")
    w, wc = counter("write", "WRITE_SIZE")
    hits, _ = counter("tcc", "TCC_HIT_sum")
    miss, _ = counter("tcc", "TCC_MISS_sum")
    # the 1 GiB copy kernel's launches: the largest copy dispatches
    cf = statistics.median([v for v in fc if v > 0.25 * probe_kib])
    cw = statistics.median([v for v in wc if v > 0.5 * probe_kib])
    fs, ws = probe_kib / cf, probe_kib / cw
    fk, wk = statistics.mean(f), statistics.mean(w)
    traffic = int(round((fk * fs + wk * ws) * 1024))
    tr = [(float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e6
          for r in rows("trace", "kernel_trace.csv") if ksub in r["Kernel_Name"]]
    avg_ms = statistics.mean(tr)
    h, m = statistics.mean(hits), statistics.mean(miss)
    rec = {
        "workload": "Wan2.1-14B clustered, 1x40x75600, d128, 128x128 blocks, 15.0% density",
        "kernel": "attn_ppx_128_128",
        "kernel_sources_sha256": attn_sources_sha256(),
        "dispatches_counted": len(f),
        "fetch_kib_per_launch": round(fk, 2), "write_kib_per_launch": round(wk, 2),
        "copy_probe_kib": probe_kib, "copy_fetch_kib": cf, "copy_write_kib": cw,
        "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
        "traffic_bytes_per_launch": traffic, "algorithmic_bytes_per_launch": 3097067520,
        "tcc_hit_per_launch": int(h), "tcc_miss_per_launch": int(m),
        "l2_hit_rate": round(h / (h + m), 4),
        "trace_launches": len(tr), "trace_avg_ms": round(avg_ms, 4),
        "achieved_hbm_gbs": round(traffic / (avg_ms * 1e-3) / 1e9, 1),
        "commands": [
            "export TMPDIR=/tmp",
            "rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o trace -- python3 bench.py "
            "--steps 1 --warmup 0 --no-cpu-baseline --headline-only",
            "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o fetch -- python3 bench.py --steps 1 "
            "--warmup 0 --no-cpu-baseline --headline-only --copy-probe-mib 1024",
            "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o write -- python3 bench.py --steps 1 "
            "--warmup 0 --no-cpu-baseline --headline-only --copy-probe-mib 1024",
            "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum --output-format csv -d DIR/tcc -o tcc -- python3 bench.py "
            "--steps 1 --warmup 0 --no-cpu-baseline --headline-only",
            "python3 bench.py --summarize-profile DIR",
        ],
    }
    path = os.path.join(ROOT, "profiles", "attn_wan14b_clustered_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def stage1_record(res):
    """The adaptive skip's statistics and decision for WaveAlign stage 1 (the
    pass's bsa_stage1_decide output), or None when it did not run."""
    if res.stage1_stats is None:
        return None
    from block_sparse_attention_mask_amd import api
    st = res.stage1_stats.cpu().numpy()
    rec = {n: round(float(v), 6) for n, v in zip(api.STAGE1_STAT_NAMES, st)}
    rec["run"] = bool(rec["run"])
    return rec


def workload_name(cfg):
    return {
        "clustered": "Wan2.1-14B 720p video DiT self-attention, clustered+permuted block-sparse "
                     "(1x40x75600, d128, 128x128 blocks, cumulative mass 0.9)",
        "importance_sampled": "Wan2.1-14B shape, group-shared importance-sampled blocks with log-weights",
        "video_threshold": "Wan2.1-1.3B video DiT shape, threshold map T<=p (1x12x32760)",
        "llm_prefill": "LLaMA-3.1-8B prefill shape, causal GQA static block pattern (32q/8kv x 65536)",
        "tiny": "tiny 1x2x1024 d64, 64x64 blocks, 25% random mask",
    }[cfg]


def stage_times(pipeline, dw, args, torch):
    from block_sparse_attention_mask_amd import api
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    torch.cuda.synchronize()
    ev[0].record(s)
    row_ptr, col, lw = api.build_csr(dw.mask, dw.T, dw.p, dw.lw_map, dw.nQB, dw.force_diag)
    ev[1].record(s)
    q, k, pq, pk = dw.q, dw.k, None, None
    if dw.permuted:
        pq = api.perm_from_labels(dw.labels_q, dw.n_clusters)
        pk = api.perm_from_labels(dw.labels_k, dw.n_clusters)
        k = api.permute_rows(dw.k, pk)
    v = api.transpose_rows(dw.v, pk, ld=dw.nQB * dw.block)
    ev[2].record(s)
    row_perm = None
    if api.spectral_supported(dw.nQB, dw.nQB):
        dec, _ = api.stage1_decide(row_ptr, col, dw.B * dw.Hq, dw.nQB, dw.nQB, dw.N, dw.d, dw.block, 10)
        row_perm, _ = api.spectral_order(row_ptr, col, dw.B * dw.Hq, dw.nQB, dw.nQB, 10, enable=dec)
    share = kv_share_ok(dw, row_ptr, col, lw)
    ev[3].record(s)
    order2 = None
    if not share and dw.block == 128:
        order, order2 = api.schedule_pairs(row_ptr, col, dw.B, dw.Hq, dw.Hkv, dw.nQB, args.wave_rows, args.n_xcd,
                                           lw=lw, row_perm=row_perm)
    else:
        order = api.schedule(row_ptr, dw.B, dw.Hq, dw.Hkv, dw.nQB, args.wave_rows, args.n_xcd, row_perm=row_perm,
                             head_step=2 if share else 1, col=col)
    ev[4].record(s)
    api.attn_fwd(q, k, v, row_ptr, col, dw.block, lw=lw, order=order, scatter_perm_q=pq,
                 gather_perm_q=pq, causal=dw.causal, v_dim_major=True, kv_share=share, order2=order2)
    ev[5].record(s)
    torch.cuda.synchronize()
    names = ["mask_to_csr", "perm_k_gather_and_v_transpose", "stage1_adaptive_skip", "schedule",
             "attention_fused_gather_scatter"]
    return {n: round(ev[i].elapsed_time(ev[i + 1]), 4) for i, n in enumerate(names)}


def row_set(w, perm_q, seed):
    """The measurement protocol's row set, as flat (b*Hq + h)*N + t rows with
    t in original order: for every (b, h, query block) the first and the last
    real row of the block in the order the kernel sees (mapped back through
    perm_q when permuted), and per (b, h) one seeded random whole block and
    the whole tail block."""
    rng = np.random.default_rng(seed)
    nb, B = w.nQB, w.block
    firsts = np.arange(nb, dtype=np.int64) * B
    lasts = np.minimum(firsts + B, w.N) - 1
    out = []
    for bh in range(w.B * w.Hq):
        rb = int(rng.integers(0, nb))
        pos = np.unique(np.concatenate([firsts, lasts, np.arange(rb * B, min(w.N, (rb + 1) * B)),
                                        np.arange((nb - 1) * B, w.N)]))
        t = perm_q[bh][pos].astype(np.int64) if perm_q is not None else pos
        out.append(bh * w.N + t)
    return np.unique(np.concatenate(out))


def rows_pairs(w, rp, col, rows, perm_q):
    """Allowed (query, key) pairs of each of the given rows (flat original
    indices), from the CSR the oracle built."""
    from block_sparse_attention_mask_amd import metrics
    bh, t = rows // w.N, rows % w.N
    if perm_q is not None:
        inv = np.empty_like(perm_q)
        for h in range(perm_q.shape[0]):
            inv[h][perm_q[h]] = np.arange(w.N, dtype=perm_q.dtype)
        pos = inv[bh, t].astype(np.int64)
    else:
        pos = t
    u = pos // w.block
    r = bh * w.nQB + u
    if not w.causal:
        nq = np.minimum(w.block, w.N - u * w.block)
        return metrics.pairs_per_row(rp, col, w.N, w.block, False)[r] // nq
    rp64 = np.asarray(rp, dtype=np.int64)
    out = np.empty(len(rows), dtype=np.int64)
    for i in range(len(rows)):
        tot = 0
        for e in range(rp64[r[i]], rp64[r[i] + 1]):
            v = int(col[e])
            if v < u[i]:
                tot += min(w.block, w.N - v * w.block)
            elif v == u[i]:
                tot += int(pos[i]) - int(u[i]) * w.block + 1
        out[i] = tot
    return out


def host_cpu():
    """The host's CPU model (first "model name" of /proc/cpuinfo) and the
    number of CPUs the OS reports, for the CPU baseline's record."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def oracle_leg(w, gpu_out, gpu_lse, gpu_csr, torch, seed=1234):
    """The CPU reference checker (fp64, every host thread) on the measurement
    protocol's row set: its own CSR and permutations from the workload's
    inputs, then every sampled row.  Reports the CPU rate in effective TFLOPS
    (same 4*d per allowed pair), the CSR's bit-exactness against the GPU's,
    and max-abs / mean-abs of the GPU output (and the LSE error) on exactly
    those rows."""
    import oracle
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    t0 = time.perf_counter()
    orp, ocol, olw = oracle.build_csr(w.mask, w.T, w.p, w.lw_map, w.nQB, w.force_diag)
    pq = oracle.perm_from_labels(w.labels_q, w.n_clusters) if w.permuted else None
    pk = oracle.perm_from_labels(w.labels_k, w.n_clusters) if w.permuted else None
    t_prep = time.perf_counter() - t0
    grp, gcol = gpu_csr
    csr_exact = bool(np.array_equal(np.asarray(grp), orp) and np.array_equal(np.asarray(gcol), ocol))
    rows = row_set(w, pq, seed)
    t1 = time.perf_counter()
    ref_o, ref_l = oracle.attn_rows(w.q, w.k, w.v, orp, ocol, olw, w.block, rows, pq, pk, w.causal)
    dt = time.perf_counter() - t1
    pairs = float(rows_pairs(w, orp, ocol, rows, pq).sum())
    idx = torch.from_numpy(rows).to(gpu_out.device)
    sel = gpu_out.reshape(-1, w.d).index_select(0, idx)
    if sel.dtype != torch.bfloat16:   # bf16 bit patterns held in an int16 tensor
        sel = sel.view(torch.bfloat16)
    got = sel.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref_o)
    rec = {"value": round(4.0 * w.d * pairs / dt / 1e12, 6), "unit": "TFLOPS", "cores": cores, "kind": "oracle",
           "sample": "the measurement protocol's row set: per (head, query block) the first and last real row, "
                     "per head one seeded random whole block and the tail block; %d of %d query rows, fp64 "
                     "dense-masked oracle with its own CSR, %.1f s" % (len(rows), w.B * w.Hq * w.N, dt),
           "seconds": round(dt, 3), "rows": int(len(rows)), "rows_per_s": round(len(rows) / dt, 1),
           "extrapolated_full_seconds": round(dt * w.B * w.Hq * w.N / len(rows), 1),
           "oracle_csr_and_perm_seconds": round(t_prep, 3),
           "host": host_cpu(),
           "csr_bit_exact": csr_exact,
           "max_abs": float(err.max()), "mean_abs": float(err.mean())}
    if gpu_lse is not None:
        gl = gpu_lse.reshape(-1).index_select(0, idx).cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_l)
        rec["lse_max_abs"] = float(np.abs(gl[fin] - ref_l[fin]).max()) if fin.any() else 0.0
        rec["lse_inf_match"] = bool(np.all(np.isneginf(gl[~fin])))
    rec["within_tolerance"] = bool(rec["max_abs"] <= 2e-2 and rec["mean_abs"] <= 2e-3 and csr_exact)
    return rec


def workload_line(cfg, args, torch, with_oracle=True):
    """One page-shaped workload besides the headline: the attention launch
    alone (10 warm-up calls, median of 50, one after an L2/MALL flush), its
    effective TFLOPS and fraction of the bf16 peak, and the oracle leg on the
    same output."""
    from block_sparse_attention_mask_amd import metrics, pipeline
    import synth
    t0 = time.time()
    w = synth.CONFIGS[cfg]()
    log("generated %s in %.1fs" % (cfg, time.time() - t0))
    dw = pipeline.to_device(w, torch.device("cuda"))
    res = pipeline.forward(dw, n_xcd=args.n_xcd, wave_rows=args.wave_rows, overlap=True, want_lse=True)
    torch.cuda.synchronize()
    rp = res.row_ptr.cpu().numpy()
    nnz = int(rp[-1])
    col = res.col[:nnz].cpu().numpy()
    pairs = metrics.count_pairs(rp, col, w.N, w.block, w.causal)
    flop = 4.0 * w.d * pairs
    solo = attention_alone(dw, args, torch)
    tf = flop / (solo["median_ms"] * 1e-3) / 1e12
    line = {"workload": workload_name(cfg),
            "shape": {"batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "seq_len": w.N, "head_dim": w.d,
                      "block": w.block, "causal": bool(w.causal), "permuted": bool(w.permuted),
                      "log_weights": w.lw_map is not None},
            "nnz_blocks": nnz, "block_density": round(nnz / float(w.R * w.nKB), 5), "allowed_pairs": int(pairs),
            "effective_gflop": round(flop / 1e9, 3),
            "kernel": attn_kernel_name(w.block, w.d, res.kv_share, res.order2 is not None),
            "kv_share": bool(res.kv_share),
            "kernel_alone_median50_ms": solo["median_ms"], "l2_flushed_ms": solo["flushed_ms"],
            "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "stage1_adaptive_skip": stage1_record(res)}
    log("%s: kernel %.3f ms (median of 50) -> %.1f TFLOPS" % (cfg, solo["median_ms"], tf))
    if with_oracle:
        line["cpu_baseline"] = oracle_leg(w, res.out, res.lse, (rp, col), torch)
        line["within_tolerance"] = line["cpu_baseline"]["within_tolerance"]
        log("%s oracle leg: %s" % (cfg, {k: v for k, v in line["cpu_baseline"].items() if k != "sample"}))
    del dw, res
    return line


if __name__ == "__main__":
    main()
