"""Seeded synthetic inputs for block-sparse attention workloads.

This module is test and benchmark infrastructure, not part of the shipped
package: the GPU path's tests and benchmark and the CPU reference checker's
tests draw their inputs from it.  It only draws random numbers and lays out the *inputs* of
the path (bf16 Q/K/V bit patterns, block masks, threshold maps, per-block
log-weight maps, cluster labels).  It contains none of the path's own
arithmetic: no CSR construction, no permutation, no schedule, no attention.

Every tensor is drawn from numpy ``Generator(Philox)`` streams spawned from a
``SeedSequence(seed)``, one stream per (tensor, head), as float32, then rounded
to bfloat16 (round-to-nearest-even) and stored as uint16 bit patterns.

Workload shapes follow the pages:

* tiny: 1x2x1024, d=64, 64x64 blocks, random 25 % block mask.
* video DiT 1.3B shape: 12 heads, N = 32760 = 21 latent frames x 30x52
  patches (ScalingAttention, experimental setup table), threshold map T with
  mask M = I(T <= p) (ScalingAttention, section 5.2, Eq. 2).
* video DiT 14B shape: 40 heads, N = 75600 = 21 frames x 3600 tokens
  (InstaGen, Experiments: Models), clustered Q/K permuted by cluster label
  (permuted block-sparse attention), KV blocks kept to cumulative mass 0.9.
* importance sampled: same shape, per query cluster an exact top-8 set plus 8
  blocks drawn by systematic PPS with PPSWOR inclusion probabilities
  (InstaGen section 3.2.1 Eq. 4 and Algorithm 1), carrying -ln(pi) as an
  additive per-block log-weight (Algorithm 1, Horvitz-Thompson weights).
* LLM prefill: 32 query / 8 KV heads, N = 65536, causal static pattern of a
  4-block local window, stride-16 same-position blocks and the first block
  (INTRA, Scatter/Gather block-level instantiation).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_THREADS = 8


# --------------------------------------------------------------------------
# bf16 helpers (bit patterns in uint16)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 with round-to-nearest-even; returns uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.Philox(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal_heads(seed: int, H: int, N: int, d: int, fn=None) -> np.ndarray:
    """[H][N][d] bf16 bits; head h uses its own stream.  ``fn(h, x, rng)`` may
    add structure to the float32 draw before rounding."""
    out = np.empty((H, N, d), dtype=np.uint16)
    gens = _streams(seed, H)

    def one(h):
        x = gens[h].standard_normal((N, d), dtype=np.float32)
        if fn is not None:
            x = fn(h, x, gens[h])
        out[h] = f32_to_bf16_bits(x)

    with ThreadPoolExecutor(min(_THREADS, H)) as ex:
        list(ex.map(one, range(H)))
    return out


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    block: int
    q: np.ndarray            # uint16 [B][Hq][N][d]
    k: np.ndarray            # uint16 [B][Hkv][N][d]
    v: np.ndarray            # uint16 [B][Hkv][N][d]
    mask: Optional[np.ndarray] = None     # uint8  [R][nKB], R = B*Hq*nQB
    T: Optional[np.ndarray] = None        # float32 [R][nKB]
    p: float = 0.0
    lw_map: Optional[np.ndarray] = None   # float32 [R][nKB]
    labels_q: Optional[np.ndarray] = None  # int32 [B*Hq][N]
    labels_k: Optional[np.ndarray] = None  # int32 [B*Hkv][N]
    n_clusters: int = 0
    causal: bool = False
    force_diag: bool = True
    info: dict = field(default_factory=dict)

    @property
    def nQB(self) -> int:
        return -(-self.N // self.block)

    @property
    def nKB(self) -> int:
        return self.nQB

    @property
    def R(self) -> int:
        return self.B * self.Hq * self.nQB

    @property
    def permuted(self) -> bool:
        return self.labels_q is not None


# --------------------------------------------------------------------------
# tiny: random 25 % block mask with the diagonal kept
# --------------------------------------------------------------------------
def tiny(seed: int = 1, B: int = 1, H: int = 2, N: int = 1024, d: int = 64, block: int = 64,
         density: float = 0.25) -> Workload:
    nb = -(-N // block)
    q = _normal_heads(seed * 1000 + 1, B * H, N, d).reshape(B, H, N, d)
    k = _normal_heads(seed * 1000 + 2, B * H, N, d).reshape(B, H, N, d)
    v = _normal_heads(seed * 1000 + 3, B * H, N, d).reshape(B, H, N, d)
    rng = np.random.Generator(np.random.Philox(np.random.SeedSequence(seed * 1000 + 4)))
    per_head = int(round(density * nb * nb))
    extra = per_head - nb
    mask = np.zeros((B * H, nb, nb), dtype=np.uint8)
    off = np.array([(u, w) for u in range(nb) for w in range(nb) if u != w], dtype=np.int64)
    for bh in range(B * H):
        mask[bh, np.arange(nb), np.arange(nb)] = 1
        if extra > 0:
            pick = rng.choice(len(off), size=extra, replace=False)
            mask[bh, off[pick, 0], off[pick, 1]] = 1
    return Workload("tiny", B, H, H, N, d, block, q, k, v, mask=mask.reshape(-1, nb),
                    info={"per_head_blocks": per_head})


# --------------------------------------------------------------------------
# video DiT (Wan2.1-1.3B shape): threshold map with spatio-temporal bands
# --------------------------------------------------------------------------
def video_threshold(seed: int = 2, H: int = 12, frames: int = 21, frame_tokens: int = 1560,
                    row_tokens: int = 52, d: int = 128, block: int = 128,
                    density: float = 0.15) -> Workload:
    N = frames * frame_tokens
    nb = -(-N // block)
    comp = _streams(seed * 1000 + 9, 2 * H)
    # one shared component per (head, frame) for Q and K, another for V
    cqk = [comp[h].standard_normal((frames, d), dtype=np.float32) for h in range(H)]
    cv = [comp[H + h].standard_normal((frames, d), dtype=np.float32) for h in range(H)]
    frame_of = (np.arange(N) // frame_tokens).astype(np.int64)
    a = np.float32(math.sqrt(0.75))

    def add(c):
        return lambda h, x, _g: a * x + np.float32(0.5) * c[h][frame_of]

    q = _normal_heads(seed * 1000 + 1, H, N, d, add(cqk))[None]
    k = _normal_heads(seed * 1000 + 2, H, N, d, add(cqk))[None]
    v = _normal_heads(seed * 1000 + 3, H, N, d, add(cv))[None]

    first = np.arange(nb) * block
    f = first // frame_tokens
    y = (first % frame_tokens) // row_tokens
    df = np.abs(f[:, None] - f[None, :]).astype(np.float32)
    dy = np.abs(y[:, None] - y[None, :]).astype(np.float32)
    base = (np.float32(0.6) * np.minimum(np.float32(1), df / np.float32(4))
            + np.float32(0.4) * np.minimum(np.float32(1), dy / np.float32(15)))
    T = np.empty((H, nb, nb), dtype=np.float32)
    gens = _streams(seed * 1000 + 5, H)
    for h in range(H):
        xi = gens[h].random((nb, nb), dtype=np.float32)
        far = gens[h].random((nb, nb), dtype=np.float32) < np.float32(0.03)
        xi2 = gens[h].random((nb, nb), dtype=np.float32)
        t = base + np.float32(0.05) * xi
        T[h] = np.where(far, np.float32(0.05) * xi2, t).astype(np.float32)
    target = int(round(density * H * nb * nb))
    flat = np.sort(T.reshape(-1))
    p = float(flat[target - 1])
    return Workload("video_threshold", 1, H, H, N, d, block, q, k, v, T=T.reshape(-1, nb), p=p,
                    info={"target_entries": target})


# --------------------------------------------------------------------------
# clustered, permuted workloads (Wan2.1-14B shape)
# --------------------------------------------------------------------------
def _block_composition(sizes: np.ndarray, N: int, block: int) -> np.ndarray:
    """W[u][c] = number of tokens of cluster c that fall in block u when the
    tokens are laid out cluster after cluster (sizes in cluster order)."""
    nb = -(-N // block)
    C = len(sizes)
    ends = np.cumsum(sizes)
    starts = ends - sizes
    bs = np.arange(nb) * block
    be = np.minimum(bs + block, N)
    lo = np.maximum(bs[:, None], starts[None, :])
    hi = np.minimum(be[:, None], ends[None, :])
    return np.maximum(hi - lo, 0).astype(np.float64).reshape(nb, C)


def _mass_T(Wc: np.ndarray, G: np.ndarray, scale: float, nvec: np.ndarray) -> np.ndarray:
    """Exclusive cumulative normalised block mass in descending-mass order
    (ties to the lower block index); rows are query blocks."""
    qbar = Wc / Wc.sum(1, keepdims=True)
    s = (qbar @ G @ qbar.T) * scale
    s = s - s.max(1, keepdims=True)
    mass = nvec[None, :] * np.exp(s)
    mass = mass / mass.sum(1, keepdims=True)
    nb = mass.shape[1]
    order = np.lexsort((np.broadcast_to(np.arange(nb), mass.shape), -mass), axis=1)
    sm = np.take_along_axis(mass, order, 1)
    exc = np.cumsum(sm, 1) - sm
    T = np.empty_like(mass)
    np.put_along_axis(T, order, exc, 1)
    return T


def clustered(seed: int = 3, H: int = 40, N: int = 75600, d: int = 128, block: int = 128,
              C: int = 64, mass_p: float = 0.9, target_density: float = 0.15,
              sigma: Optional[float] = None) -> Workload:
    """Clustered Q/K with per-head Gaussian centroids mu_c = sigma * g_c.

    Tokens carry labels l_t ~ U{0..C-1}; q_t = mu_{l_t} + z_t, k_t = mu_{l_t} + z'_t,
    v ~ N(0, 1).  Query/key blocks are those of the sequence permuted by
    cluster label (stable).  The block mass proxy is the centroid score of the
    blocks' cluster mixtures, mass(u, v) ~ |v| exp(scale * qbar_u . kbar_v); T
    holds the exclusive cumulative mass of each row in descending order, so
    that T <= 0.9 keeps the top blocks up to cumulative mass 0.9.  sigma is
    found by bisection so that global density (forced diagonal included) is
    close to ``target_density``.
    """
    nb = -(-N // block)
    gens = _streams(seed * 1000 + 7, H)
    labels = np.empty((H, N), dtype=np.int32)
    gdir = np.empty((H, C, d), dtype=np.float32)
    for h in range(H):
        labels[h] = gens[h].integers(0, C, size=N, dtype=np.int32)
        gdir[h] = gens[h].standard_normal((C, d), dtype=np.float32)
    sizes = np.stack([np.bincount(labels[h], minlength=C) for h in range(H)])
    Wc = [_block_composition(sizes[h], N, block) for h in range(H)]
    G0 = [gdir[h].astype(np.float64) @ gdir[h].astype(np.float64).T for h in range(H)]
    nvec = np.minimum(block, N - np.arange(nb) * block).astype(np.float64)
    scale = 1.0 / math.sqrt(d)
    eye = np.eye(nb, dtype=bool)

    def density(sig):
        tot = 0
        for h in range(H):
            T = _mass_T(Wc[h], G0[h] * sig * sig, scale, nvec)
            tot += int(((T <= mass_p) | eye).sum())
        return tot / (H * nb * nb)

    if sigma is None:
        lo, hi = 0.05, 2.0   # density decreases as sigma grows
        for _ in range(24):
            mid = 0.5 * (lo + hi)
            if density(mid) > target_density:
                lo = mid
            else:
                hi = mid
        sigma = 0.5 * (lo + hi)
    T = np.empty((H, nb, nb), dtype=np.float32)
    for h in range(H):
        T[h] = _mass_T(Wc[h], G0[h] * sigma * sigma, scale, nvec).astype(np.float32)

    mu = (gdir * np.float32(sigma)).astype(np.float32)

    def add_mu(h, x, _g):
        x += mu[h][labels[h]]
        return x

    q = _normal_heads(seed * 1000 + 1, H, N, d, add_mu)[None]
    k = _normal_heads(seed * 1000 + 2, H, N, d, add_mu)[None]
    v = _normal_heads(seed * 1000 + 3, H, N, d)[None]
    dens = float((((T <= np.float32(mass_p)) | eye[None]).sum()) / (H * nb * nb))
    return Workload("clustered", 1, H, H, N, d, block, q, k, v, T=T.reshape(-1, nb), p=float(mass_p),
                    labels_q=labels, labels_k=labels.copy(), n_clusters=C,
                    info={"sigma": float(sigma), "density": dens, "cluster_sizes": sizes})


def _water_fill(s: np.ndarray, m: float) -> np.ndarray:
    """PPSWOR inclusion probabilities pi_j = min(1, lam * s_j) with sum = m
    (InstaGen Eq. 4).  s > 0, len(s) > m."""
    order = np.argsort(-s, kind="stable")
    ss = s[order]
    n = len(ss)
    pi = None
    for k in range(0, int(m) + 1):   # k = number of capped entries
        rest = ss[k:].sum()
        lam = (m - k) / rest
        if k < n and lam * ss[k] <= 1.0 + 1e-12 and (k == 0 or lam * ss[k - 1] >= 1.0 - 1e-12):
            pi_sorted = np.minimum(1.0, lam * ss)
            pi_sorted[:k] = 1.0
            pi = np.empty(n)
            pi[order] = pi_sorted
            break
    if pi is None:
        raise RuntimeError("water-filling failed")
    return pi


def importance_sampled(seed: int = 4, H: int = 40, N: int = 75600, d: int = 128, block: int = 128,
                       C: int = 64, m_exact: int = 8, m_sample: int = 8,
                       sigma: Optional[float] = None) -> Workload:
    """Group-shared importance sampling over KV blocks (InstaGen Algorithm 1 at
    block granularity): for every query cluster g, the exact set E_g is the
    top ``m_exact`` blocks by estimated mass; the residual blocks get
    PPSWOR probabilities pi = min(1, lam * mass) summing to ``m_sample``; a
    systematic PPS sample (ascending block order, one uniform offset per
    cluster) picks the sampled blocks, each with log-weight -ln(pi).  Every
    query block whose first token belongs to cluster g shares that list.  The
    diagonal block is forced by the mask builder; its log-weight is 0."""
    base = clustered(seed=seed, H=H, N=N, d=d, block=block, C=C, sigma=sigma)
    nb = base.nQB
    sigma = base.info["sigma"]
    sizes = base.info["cluster_sizes"]
    gens = _streams(seed * 1000 + 11, H)
    rng_g = _streams(seed * 1000 + 7, H)
    gdir = np.empty((H, C, d), dtype=np.float32)
    for h in range(H):   # same draws as clustered(): labels first, then directions
        rng_g[h].integers(0, C, size=N, dtype=np.int32)
        gdir[h] = rng_g[h].standard_normal((C, d), dtype=np.float32)
    scale = 1.0 / math.sqrt(d)
    nvec = np.minimum(block, N - np.arange(nb) * block).astype(np.float64)
    mask = np.zeros((H, nb, nb), dtype=np.uint8)
    lw = np.zeros((H, nb, nb), dtype=np.float32)
    n_sampled = 0
    for h in range(H):
        Wc = _block_composition(sizes[h], N, block)
        mu = gdir[h].astype(np.float64) * sigma
        kbar = (Wc / Wc.sum(1, keepdims=True)) @ mu          # [nb][d]
        ends = np.cumsum(sizes[h])
        first_cluster = np.searchsorted(ends, np.arange(nb) * block, side="right")
        for g in np.unique(first_cluster):
            sc = (kbar @ mu[g]) * scale
            mass = nvec * np.exp(sc - sc.max())
            order = np.lexsort((np.arange(nb), -mass))
            exact = np.sort(order[:m_exact])
            resid = np.sort(order[m_exact:])
            pi = _water_fill(mass[resid], float(m_sample))
            cum = np.concatenate([[0.0], np.cumsum(pi)])
            u0 = gens[h].random()
            pts = u0 + np.arange(m_sample)
            idx = np.searchsorted(cum, pts, side="right") - 1
            sel = resid[idx]
            rows = np.nonzero(first_cluster == g)[0]
            mask[h][np.ix_(rows, exact)] = 1
            mask[h][np.ix_(rows, sel)] = 1
            lw[h][np.ix_(rows, sel)] = (-np.log(pi[idx])).astype(np.float32)
            n_sampled += len(sel) * len(rows)
        lw[h][np.arange(nb), np.arange(nb)] = 0.0
    return Workload("importance_sampled", 1, H, H, N, d, block, base.q, base.k, base.v,
                    mask=mask.reshape(-1, nb), lw_map=lw.reshape(-1, nb),
                    labels_q=base.labels_q, labels_k=base.labels_k, n_clusters=C,
                    info={"sigma": sigma, "sampled_entries": n_sampled})


# --------------------------------------------------------------------------
# LLM prefill: causal static block pattern, GQA
# --------------------------------------------------------------------------
def prefill_pattern(nb: int, window: int = 4, stride: int = 16) -> np.ndarray:
    """uint8 [nb][nb]: row u keeps blocks u-window+1..u, every block v < u with
    v = u (mod stride), and block 0."""
    m = np.zeros((nb, nb), dtype=np.uint8)
    for u in range(nb):
        m[u, max(0, u - window + 1):u + 1] = 1
        m[u, u % stride:u:stride] = 1
        m[u, 0] = 1
    return m


def llm_prefill(seed: int = 5, Hq: int = 32, Hkv: int = 8, N: int = 65536, d: int = 128,
                block: int = 128) -> Workload:
    nb = -(-N // block)
    q = _normal_heads(seed * 1000 + 1, Hq, N, d)[None]
    k = _normal_heads(seed * 1000 + 2, Hkv, N, d)[None]
    v = _normal_heads(seed * 1000 + 3, Hkv, N, d)[None]
    pat = prefill_pattern(nb)
    mask = np.ascontiguousarray(np.broadcast_to(pat, (Hq, nb, nb))).reshape(-1, nb)
    return Workload("llm_prefill", 1, Hq, Hkv, N, d, block, q, k, v, mask=mask, causal=True)


# --------------------------------------------------------------------------
# small random cases for parity tests
# --------------------------------------------------------------------------
def random_case(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int, block: int,
                density: float = 0.3, causal: bool = False, permute: bool = False,
                log_weights: bool = False, n_clusters: int = 5, use_T: bool = False,
                q_scale: float = 1.0) -> Workload:
    """Small random workload for element-by-element parity: random block mask
    (or threshold map), optional labels, optional log-weight map."""
    nb = -(-N // block)
    R = B * Hq * nb
    gens = _streams(seed, 8)
    f = lambda g, H: f32_to_bf16_bits(g.standard_normal((B, H, N, d), dtype=np.float32) *
                                      np.float32(q_scale)).reshape(B, H, N, d)
    q = f(gens[0], Hq)
    k = f(gens[1], Hkv)
    v = f32_to_bf16_bits(gens[2].standard_normal((B, Hkv, N, d), dtype=np.float32))
    w = Workload("random", B, Hq, Hkv, N, d, block, q, k, v, causal=causal)
    if use_T:
        w.T = gens[3].random((R, nb), dtype=np.float32)
        w.p = float(density)
    else:
        w.mask = (gens[3].random((R, nb)) < density).astype(np.uint8)
    if log_weights:
        w.lw_map = gens[4].uniform(-3.0, 3.0, size=(R, nb)).astype(np.float32)
    if permute:
        w.labels_q = gens[5].integers(0, n_clusters, size=(B * Hq, N), dtype=np.int32)
        w.labels_k = gens[6].integers(0, n_clusters, size=(B * Hkv, N), dtype=np.int32)
        w.n_clusters = n_clusters
    return w


# --------------------------------------------------------------------------
# Token-level computational query sets: index maps only
# --------------------------------------------------------------------------
def _lists_to_csr(qsets, ksets, BQ):
    C = len(qsets)
    q_idx = np.full((C, BQ), -1, dtype=np.int32)
    for i, qs in enumerate(qsets):
        q_idx[i, :len(qs)] = qs
    kv_ptr = np.zeros(C + 1, dtype=np.int32)
    kv_ptr[1:] = np.cumsum([len(k) for k in ksets])
    kv_idx = np.concatenate(ksets).astype(np.int32) if C else np.zeros(0, np.int32)
    return q_idx, kv_ptr, kv_idx


def cqs_scatter(N: int, R: int = 8, BQ: int = 64, causal: bool = False):
    """INTRA Scatter (sections 4.2 and 4.8): relay group r holds the tokens
    r, r + R, r + 2R, ... (one token of every R-token neighbourhood); each
    query set is BQ consecutive members of one group and its keys are the
    group's members (when causal, only those up to the set's last query).
    Returns (q_idx [C][BQ], kv_ptr [C+1], kv_idx) for one head."""
    qsets, ksets = [], []
    for r in range(R):
        members = np.arange(r, N, R)
        for b0 in range(0, len(members), BQ):
            qsets.append(members[b0:b0 + BQ])
            ksets.append(members[:b0 + BQ] if causal else members)
    return _lists_to_csr(qsets, ksets, BQ)


def cqs_gather1(N: int, R: int = 8, BQ: int = 64, causal: bool = False):
    """INTRA Gather 1 (appendix: the repeated-segment token grouping of the
    token-level benchmarks; the cyclic Gather of the relay analysis), read as:
    the sequence splits into segments of R consecutive tokens (the
    neighbourhoods Scatter takes one token from), and segment p joins group
    p mod R, so group b holds the segments b, b + R, b + 2R, ...  Each query
    set is BQ consecutive members of one group and its keys are the group's
    members (when causal, only those up to the set's last query).  Returns
    (q_idx [C][BQ], kv_ptr [C+1], kv_idx) for one head."""
    qsets, ksets = [], []
    seg = np.arange(N) // R
    for b in range(R):
        members = np.nonzero(seg % R == b)[0]
        for b0 in range(0, len(members), BQ):
            qsets.append(members[b0:b0 + BQ])
            ksets.append(members[:b0 + BQ] if causal else members)
    return _lists_to_csr(qsets, ksets, BQ)


def cqs_gather0(H: int, W: int):
    """INTRA Gather 0 (appendix, sparse pattern index functions): query set i
    is the 8x8 patch (r, c) = divmod(i, W / 8) of an H x W token image
    (row-major); its keys are the 16 x 16 window with top-left corner
    (clamp(8r - 4, 0, H - 16), clamp(8c - 4, 0, W - 16)), taken as four
    64-key tiles of four rows of 16 keys.  Returns (q_idx [C][64], kv_ptr
    [C+1], kv_idx) for one head."""
    assert H >= 16 and W >= 16 and H % 8 == 0 and W % 8 == 0
    qsets, ksets = [], []
    for i in range((H // 8) * (W // 8)):
        r, c = divmod(i, W // 8)
        il = np.arange(64)
        qsets.append((8 * r + il // 8) * W + 8 * c + il % 8)
        r0 = min(max(8 * r - 4, 0), H - 16)
        c0 = min(max(8 * c - 4, 0), W - 16)
        jl = np.arange(256)
        ksets.append((r0 + jl // 16) * W + c0 + jl % 16)
    return _lists_to_csr(qsets, ksets, 64)


def cqs_token_select(seed: int, N: int, BQ: int, n_keys: int):
    """Token-level KV selection shape (MC-Sparse): the sequence (in its
    grouped order) splits into query groups of BQ consecutive tokens, and each
    group attends to its own n_keys distinct key tokens, drawn uniformly
    without replacement and listed in ascending order.  Returns (q_idx
    [C][BQ], kv_ptr [C+1], kv_idx) for one head."""
    g = _streams(seed, 1)[0]
    qsets, ksets = [], []
    for b0 in range(0, N, BQ):
        qsets.append(np.arange(b0, min(N, b0 + BQ)))
        ksets.append(np.sort(g.choice(N, size=min(n_keys, N), replace=False)))
    return _lists_to_csr(qsets, ksets, BQ)


def cqs_per_head(maps, BH: int):
    """Stacks one head's (q_idx, kv_ptr, kv_idx) for BH heads (the same sets
    in every head)."""
    q_idx, kv_ptr, kv_idx = maps
    C = q_idx.shape[0]
    nnz = int(kv_ptr[-1])
    ptr = (kv_ptr[None, :-1].astype(np.int64) + nnz * np.arange(BH)[:, None]).reshape(-1)
    kv_ptr_all = np.concatenate([ptr, [nnz * BH]]).astype(np.int32)
    return (np.broadcast_to(q_idx, (BH, C, q_idx.shape[1])).copy(), kv_ptr_all, np.tile(kv_idx, BH))


CONFIGS = {
    "tiny": tiny,
    "video_threshold": video_threshold,
    "clustered": clustered,
    "importance_sampled": importance_sampled,
    "llm_prefill": llm_prefill,
}
