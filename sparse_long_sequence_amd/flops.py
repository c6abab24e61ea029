"""Useful work of one call: allowed (query, key) pairs, FLOPs and algorithmic bytes.

Useful FLOPs count 4*D per allowed pair: 2*D for the q.k multiply-adds and
2*D for the p*v multiply-adds (LongNet page, §3.4 "Computational Complexity
and Token Dependency Analysis": two products of equal cost per attended pair).
Masked work inside edge tiles is not counted. Algorithmic bytes are Q, K, V
read once, O written once, lse written once, plus the separate global
projections (Q_g for the global rows, K_g and V_g in full).
"""
from __future__ import annotations

import numpy as np

from .workloads import LABEL_DISTANCE, Workload, etc_structure


def band_global_pairs(w: Workload) -> int:
    """Allowed pairs of the band + global pattern, summed over batch and heads.
    With packed documents (contiguous runs of positions) every piece stays
    inside a row's own document."""
    N, R = w.N, w.radius
    G = np.array(sorted(w.global_idx), dtype=np.int64)
    is_g = np.zeros(N, dtype=bool)
    is_g[G] = True
    i = np.arange(N, dtype=np.int64)
    # the run [s0, s1) of positions that a row may attend within
    s0 = np.zeros(N, dtype=np.int64)
    s1 = np.full(N, N, dtype=np.int64)
    doc = np.zeros(N, dtype=np.int64)
    if w.documents:
        off = 0
        for dn, n in enumerate(w.documents):
            s0[off:off + n], s1[off:off + n], doc[off:off + n] = off, off + n, dn
            off += n
        s0[off:], s1[off:], doc[off:] = off, N, len(w.documents)
    total = 0
    for h in range(w.H):
        d = w.dilation[h] if w.dilation else 1
        left = np.minimum(R, (i - s0) // d)
        right = np.zeros_like(i) if w.causal else np.minimum(R, (s1 - 1 - i) // d)
        cnt = left + right + 1
        if G.size:
            dl = G[None, :] - i[:, None]
            in_band = (dl % d == 0) & (np.abs(dl) <= d * R) & ((dl <= 0) if w.causal else True)
            ok = (dl <= 0) if w.causal else np.ones_like(in_band)
            same = doc[G][None, :] == doc[:, None]
            cnt = cnt + (ok & ~in_band & same).sum(axis=1)
        rows_g = (i - s0 + 1) if w.causal else (s1 - s0)
        cnt = np.where(is_g, rows_g, cnt)
        total += int(cnt.sum())
    return total * w.B


def structured_pairs(w: Workload) -> int:
    """Allowed pairs of an ETC structured workload (globals first, non-causal,
    no dilation): a global row sees every key its label row does not mask; a
    long row sees the long keys of its band inside its own context (l2l
    segment mask) and every global its label row does not mask."""
    st = etc_structure(w)
    V = st["n_labels"]
    ng, N, R = len(w.global_idx), w.N, w.radius
    masked = lambda lab: (lab != LABEL_DISTANCE) & (lab >= V)
    g_rows = int((~masked(st["glabel"][0])).sum())
    l2g = int((~masked(st["llabel"][0][ng:])).sum())
    seg = st["seg"][0].astype(np.int64)
    l2l = 0
    for i in range(ng, N):
        lo, hi = max(ng, i - R), min(N - 1, i + R)
        l2l += int((seg[lo:hi + 1] == seg[i]).sum())
    return w.B * w.H * (g_rows + l2g + l2l)


def dilated_pairs_head(w: Workload, h: int) -> int:
    """Pairs attended by all (w, r) patterns in head h of one batch row (a pair
    counted once per pattern): per segment, the kept rows of the head's offset
    attend each other (causal: a triangle)."""
    total = 0
    for (seg_w, r) in w.pairs:
        s = h % r
        for start in range(0, w.N, seg_w):
            L = min(seg_w, w.N - start)
            n = (L - s + r - 1) // r if s < L else 0
            total += n * (n + 1) // 2 if w.causal else n * n
    return total


def dilated_pairs(w: Workload) -> int:
    """Pairs attended by all (w, r) patterns (a pair counted once per pattern)."""
    return w.B * sum(dilated_pairs_head(w, h) for h in range(w.H))


def fixed_pairs(w: Workload) -> int:
    """Pairs of the fixed pattern (N a multiple of l): the own block (causal: up
    to the query) plus c summary keys of every other (causal: earlier) block."""
    l, c = w.fixed
    nb = w.N // l
    if w.causal:
        per_head = nb * l * (l + 1) // 2 + c * l * nb * (nb - 1) // 2
    else:
        per_head = nb * l * l + nb * l * (nb - 1) * c
    return per_head * w.H * w.B


def useful_pairs(w: Workload) -> int:
    if w.kind == "dilated":
        return dilated_pairs(w)
    if w.kind == "fixed":
        return fixed_pairs(w)
    if w.structure:
        return structured_pairs(w)
    return band_global_pairs(w)


def useful_flops(w: Workload) -> int:
    return 4 * w.D * useful_pairs(w)


def algorithmic_bytes(w: Workload) -> int:
    el = 2 if w.dtype == "bf16" else 4
    t = w.B * w.H * w.N * w.D * el
    b = 4 * t + w.B * w.H * w.N * 4  # q, k, v, out, lse
    if w.separate_global:
        b += 2 * t + w.B * w.H * len(w.global_idx) * w.D * el
    if w.rel_k:
        nv = w.H * (2 * w.rel_k + 1 + (4 if w.structure else 0))
        b += nv * 4 * {"scalar": 1, "vector": w.D, "both": w.D + 1}[w.rel_kind]
    if w.structure:  # the two label matrices and the segment ids
        ng = len(w.global_idx)
        b += w.B * (2 * ng * w.N + 4 * w.N)
    b += len(w.global_idx) * 4
    return b
