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

from .workloads import Workload


def band_global_pairs(w: Workload) -> int:
    """Allowed pairs of the band + global pattern, summed over batch and heads."""
    N, R = w.N, w.radius
    G = np.array(sorted(w.global_idx), dtype=np.int64)
    is_g = np.zeros(N, dtype=bool)
    is_g[G] = True
    i = np.arange(N, dtype=np.int64)
    total = 0
    for h in range(w.H):
        d = w.dilation[h] if w.dilation else 1
        # window keys i + d*m inside [0, N): m from -min(R, i//d) to min(R, (N-1-i)//d)
        left = np.minimum(R, i // d)
        right = np.zeros_like(i) if w.causal else np.minimum(R, (N - 1 - i) // d)
        cnt = left + right + 1
        if G.size:
            # globals outside the window (and not after i when causal)
            dl = G[None, :] - i[:, None]
            in_band = (dl % d == 0) & (np.abs(dl) <= d * R) & ((dl <= 0) if w.causal else True)
            ok = (dl <= 0) if w.causal else np.ones_like(in_band)
            cnt = cnt + (ok & ~in_band).sum(axis=1)
        rows_g = (i + 1) if w.causal else np.full(N, N, dtype=np.int64)
        cnt = np.where(is_g, rows_g, cnt)
        total += int(cnt.sum())
    return total * w.B


def dilated_pairs(w: Workload) -> int:
    """Pairs attended by all (w, r) patterns (a pair counted once per pattern)."""
    total = 0
    for h in range(w.H):
        for (seg_w, r) in w.pairs:
            s = h % r
            for start in range(0, w.N, seg_w):
                L = min(seg_w, w.N - start)
                n = (L - s + r - 1) // r if s < L else 0
                total += n * (n + 1) // 2 if w.causal else n * n
    return total * w.B


def useful_pairs(w: Workload) -> int:
    return dilated_pairs(w) if w.kind == "dilated" else band_global_pairs(w)


def useful_flops(w: Workload) -> int:
    return 4 * w.D * useful_pairs(w)


def algorithmic_bytes(w: Workload) -> int:
    el = 2 if w.dtype == "bf16" else 4
    t = w.B * w.H * w.N * w.D * el
    b = 4 * t + w.B * w.H * w.N * 4  # q, k, v, out, lse
    if w.separate_global:
        b += 2 * t + w.B * w.H * len(w.global_idx) * w.D * el
    if w.rel_k:
        b += w.H * (2 * w.rel_k + 1) * 4
    b += len(w.global_idx) * 4
    return b
