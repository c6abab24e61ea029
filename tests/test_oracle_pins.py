"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Nothing here re-types the oracle's own predicate or re-calls its routines to
check themselves. Each pin uses another route to the same fact:

* constructive key enumeration from the pages' wording (keys i + d*m,
  |m| <= w/2; global rows and columns) against the oracle's mask predicate;
* closed-form pair counts (w+1 keys per interior row; the ETC cost formula
  n_g(n_g+n_l) + n_l(n_g+2r+1) less the window's edge loss; LongNet's
  per-segment triangle counts) read through exp(lse) with Q = 0;
* the LongNet page's worked sparsification example (golden fixture);
* special cases that reduce to library dense attention (torch SDPA in fp64);
* plain-Python brute force on tiny inputs, including ETC's four-piece
  formulation with its two unified softmaxes and LongNet's literal
  sparsify -> attend -> scatter -> weighted-sum procedure;
* algebraic identities (mixture == joint softmax; duplicate patterns; rows
  of P sum to one).

``test_planted_mistakes_are_caught`` plants plausible mistakes in a copy of the
oracle's source, rebuilds it, and checks that every mistake fails some pin.
"""
from __future__ import annotations

import math
import os
import random
import shutil
import tempfile

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# closed forms and brute force (independent of oracle.cpp)
# ---------------------------------------------------------------------------

def count_1d(n: int, R: int, causal: bool) -> int:
    """Allowed pairs of a radius-R window on a length-n sequence."""
    if n <= 0:
        return 0
    if causal:
        if n <= R + 1:
            return n * (n + 1) // 2
        return (R + 1) * (R + 2) // 2 + (n - R - 1) * (R + 1)
    if n <= R + 1:
        return n * n
    return n * (2 * R + 1) - R * (R + 1)


def count_dilated(N: int, R: int, d: int, causal: bool) -> int:
    """Residue class c of a dilation-d window is a length ceil((N-c)/d) band."""
    return sum(count_1d((N - c + d - 1) // d, R, causal) for c in range(min(d, N)))


def count_prefix_globals(N: int, R: int, g: int) -> int:
    """Non-causal, d=1, G = {0..g-1}: global rows see N keys; a row i >= g sees
    its window plus the globals left of the window, min(g, max(0, i-R))."""
    tot = g * N
    for i in range(g, N):
        lo, hi = max(0, i - R), min(N - 1, i + R)
        tot += (hi - lo + 1) + min(g, lo)
    return tot


def longnet_row_count(N: int, pairs, h: int, i: int, causal: bool) -> int:
    tot = 0
    for (w, r) in pairs:
        s = h % r
        seg = (i // w) * w
        L = min(w, N - seg)
        if (i - seg) % r != s:
            continue
        n_seg = (L - s + r - 1) // r
        m = (i - seg - s) // r
        tot += (m + 1) if causal else n_seg
    return tot


def longnet_count(N: int, pairs, h: int, causal: bool) -> int:
    tot = 0
    for (w, r) in pairs:
        s = h % r
        for seg in range(0, N, w):
            L = min(w, N - seg)
            n = (L - s + r - 1) // r if s < L else 0
            tot += n * (n + 1) // 2 if causal else n * n
    return tot


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def bf_attend(qi, keys, K, V, bias=None):
    """Softmax attention of one query over an explicit key list (Python floats)."""
    D = len(qi)
    sc = 1.0 / math.sqrt(D)
    logits = [sc * _dot(qi, K[j]) + (bias(j) if bias else 0.0) for j in keys]
    M = max(logits)
    e = [math.exp(x - M) for x in logits]
    Z = sum(e)
    out = [sum(e[t] * V[j][c] for t, j in enumerate(keys)) / Z for c in range(D)]
    return out, M + math.log(Z)


def bf_band_head(q, k, v, G, R, d, causal, qg=None, kg=None, vg=None, relb=None, relv=None,
                 seg=None):
    """Longformer pattern by enumeration: keys i + d*m, m in [-R, R] (causal:
    [-R, 0]), inside [0, N); plus the global columns; global rows see all.
    relv ([2k+1][D]): ETC's key-side label vectors, the logit written out as
    q_i . (k_j + a_l) / sqrt(D) for same-kind pairs (bf_attend adds the
    q_i . k_j / sqrt(D) part, so the bias is the remaining q_i . a_l / sqrt(D)).
    seg: a segment id per position; keys of another segment are dropped."""
    N = len(q)
    Gs = set(G)
    outs, lses = [], []
    for i in range(N):
        if i in Gs:
            keys = [j for j in range(N) if (not causal or j <= i)]
            Q, K, V = (qg, kg, vg) if qg is not None else (q, k, v)
        else:
            steps = range(-R, 1) if causal else range(-R, R + 1)
            ks = {i + d * m for m in steps if 0 <= i + d * m < N}
            ks |= {g for g in Gs if (not causal or g <= i)}
            keys = sorted(ks)
            Q, K, V = q, k, v
        if seg is not None:
            keys = [j for j in keys if seg[j] == seg[i]]
        bias = None
        if relb is not None or relv is not None:
            kk = (len((relb if relb is not None else relv)) - 1) // 2

            def bias(j, i=i, kk=kk, Qi=Q[i]):
                if (j in Gs) != (i in Gs):
                    return 0.0
                lab = max(-kk, min(kk, j - i)) + kk
                b = relb[lab] if relb is not None else 0.0
                if relv is not None:
                    b += sum(a * x for a, x in zip(Qi, relv[lab])) / math.sqrt(len(Qi))
                return b
        o, l = bf_attend(Q[i], keys, K, V, bias)
        outs.append(o)
        lses.append(l)
    return np.array(outs), np.array(lses)


def bf_etc_four_pieces(qg_, kg_, vg_, ql, kl, vl, r, relb):
    """ETC global-local attention from its four pieces: a global query takes one
    softmax over [g2g ; g2l], a long query one over [l2g ; l2l within radius r].
    Relative labels (clipped distance) apply within g2g and l2l."""
    ng, nl = len(qg_), len(ql)
    kk = (len(relb) - 1) // 2
    D = len(ql[0])
    sc = 1.0 / math.sqrt(D)
    lab = lambda dlt: relb[max(-kk, min(kk, dlt)) + kk]
    out, lse = [], []
    for i in range(ng):
        e = [sc * _dot(qg_[i], kg_[j]) + lab(j - i) for j in range(ng)]
        e += [sc * _dot(qg_[i], kl[j]) for j in range(nl)]
        vals = list(vg_) + list(vl)
        M = max(e)
        p = [math.exp(x - M) for x in e]
        Z = sum(p)
        out.append([sum(p[t] * vals[t][c] for t in range(len(p))) / Z for c in range(D)])
        lse.append(M + math.log(Z))
    for i in range(nl):
        keys = [j for j in range(max(0, i - r), min(nl, i + r + 1))]
        e = [sc * _dot(ql[i], kg_[j]) for j in range(ng)]
        e += [sc * _dot(ql[i], kl[j]) + lab(j - i) for j in keys]
        vals = list(vg_) + [vl[j] for j in keys]
        M = max(e)
        p = [math.exp(x - M) for x in e]
        Z = sum(p)
        out.append([sum(p[t] * vals[t][c] for t in range(len(p))) / Z for c in range(D)])
        lse.append(M + math.log(Z))
    return np.array(out), np.array(lse)


def bf_longnet_head(q, k, v, pairs, h, causal):
    """LongNet's procedure as the page orders it: per pattern, sparsify each
    segment with head offset h mod r, attend densely on the sparsified rows,
    scatter back (zeros elsewhere), then mix with alpha_i = s_i / sum_j s_j."""
    N, D = len(q), len(q[0])
    sc = 1.0 / math.sqrt(D)
    Os, Ss = [], []
    for (w, r) in pairs:
        s = h % r
        Oh = [[0.0] * D for _ in range(N)]
        den = [0.0] * N
        for seg in range(0, N, w):
            L = min(w, N - seg)
            idx = list(range(seg + s, seg + L, r))
            for a, i in enumerate(idx):
                keys = idx[: a + 1] if causal else idx
                e = [math.exp(sc * _dot(q[i], k[j])) for j in keys]
                Z = sum(e)
                Oh[i] = [sum(e[t] * v[j][c] for t, j in enumerate(keys)) / Z for c in range(D)]
                den[i] = Z
        Os.append(Oh)
        Ss.append(den)
    out, lse = [], []
    for i in range(N):
        S = sum(Ss[p][i] for p in range(len(pairs)))
        if S == 0.0:
            out.append([0.0] * D)
            lse.append(-math.inf)
            continue
        out.append([sum(Ss[p][i] * Os[p][i][c] for p in range(len(pairs))) / S for c in range(D)])
        lse.append(math.log(S))
    return np.array(out), np.array(lse)


def rand_qkv(rng: np.random.Generator, B, H, N, D):
    return [rng.standard_normal((B, H, N, D)) for _ in range(3)]


def sdpa(q, k, v, causal=False):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal)
    D = q.shape[-1]
    s = torch.matmul(t[0], t[1].transpose(-1, -2).contiguous()) / math.sqrt(D)
    if causal:
        N = q.shape[-2]
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), -math.inf)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


# ---------------------------------------------------------------------------
# pins (each takes the oracle library so the planted-mistake test can reuse it)
# ---------------------------------------------------------------------------

def pin_mask_matches_enumeration(lib):
    rnd = random.Random(11)
    for _ in range(60):
        N = rnd.randint(1, 40)
        R = rnd.randint(0, N + 2)
        d = rnd.randint(1, 4)
        causal = rnd.random() < 0.5
        G = sorted(rnd.sample(range(N), rnd.randint(0, min(4, N))))
        m = oracle.mask_rows(N, G, R, d, causal, lib=lib)
        for i in range(N):
            if i in G:
                ks = {j for j in range(N) if not causal or j <= i}
            else:
                steps = range(-R, 1) if causal else range(-R, R + 1)
                ks = {i + d * s for s in steps if 0 <= i + d * s < N}
                ks |= {g for g in G if not causal or g <= i}
            assert set(np.nonzero(m[i])[0].tolist()) == ks, (N, R, d, causal, G, i)


def _count_via_lse(lib, N, G, R, dil, causal, H=1):
    z = np.zeros((1, H, N, 8))
    _, lse = oracle.attn_rows(z, z, z, G, R, dil, causal, lib=lib)
    return np.exp(lse)


def pin_counts_closed_form(lib):
    # Interior rows of a radius-R window see w+1 = 2R+1 keys (R+1 causal).
    c = _count_via_lse(lib, 200, (), 20, None, False)[0, 0]
    assert np.allclose(c[20:180], 41, rtol=0, atol=1e-9)
    assert abs(c.sum() - count_1d(200, 20, False)) < 1e-6
    c = _count_via_lse(lib, 200, (), 20, None, True)[0, 0]
    assert np.allclose(c[20:], 21, rtol=0, atol=1e-9)
    assert abs(c.sum() - count_1d(200, 20, True)) < 1e-6
    # Dilation: every residue class is an undilated band of its own length.
    for d, causal in ((2, False), (3, True), (5, False)):
        c = _count_via_lse(lib, 157, (), 7, [d], causal)
        assert abs(c.sum() - count_dilated(157, 7, d, causal)) < 1e-6
    # Prefix globals, non-causal.
    c = _count_via_lse(lib, 300, tuple(range(9)), 25, None, False)
    assert abs(c.sum() - count_prefix_globals(300, 25, 9)) < 1e-6


def pin_counts_full_workloads(lib):
    # Longformer-base workload: N=4096, R=256, G = first 64 positions.
    m = oracle.mask_rows(4096, range(64), 256, 1, False, lib=lib)
    assert int(m.sum(dtype=np.int64)) == count_prefix_globals(4096, 256, 64) == 2_522_816
    # ETC workload as one concatenated sequence: the cost formula
    # n_g(n_g+n_l) + n_l(n_g+2r+1) counts 2r+1 keys for every long row; the
    # window loses r(r+1) keys at the two ends of the long input.
    ng, nl, r = 256, 4096, 84
    m = oracle.mask_rows(ng + nl, range(ng), r, 1, False, lib=lib)
    assert int(m.sum(dtype=np.int64)) == ng * (ng + nl) + nl * (ng + 2 * r + 1) - r * (r + 1) \
        == 2_847_772
    # Char-LM workload: causal R=512, dilation 2 on a head.
    rows = [0, 1, 600, 1023, 1024, 1025, 16383]
    m = oracle.mask_rows(16384, (), 512, 2, True, rows=rows, lib=lib)
    for x, i in enumerate(rows):
        assert int(m[x].sum()) == min(i // 2, 512) + 1


def pin_longnet_counts(lib):
    pairs = ((16, 1), (32, 2), (64, 4), (96, 6))
    for N in (96, 100):
        for causal in (True, False):
            for h in range(7):
                mlt = oracle.longnet_mult_rows(N, h, pairs, causal, lib=lib)
                assert int(mlt.sum()) == longnet_count(N, pairs, h, causal)
                for i in range(N):
                    assert int(mlt[i].sum()) == longnet_row_count(N, pairs, h, i, causal)
    # The 32K-token workload, on sampled rows, and its total by closed form.
    big = ((2048, 1), (4096, 2), (8192, 4), (16384, 6), (32768, 12))
    assert sum(longnet_count(32768, big, h, True) for h in range(12)) == 839_254_020
    rows = [0, 5, 2047, 2048, 2730, 5461, 16383, 16384, 27305, 32767]
    for h in (0, 5, 11):
        mlt = oracle.longnet_mult_rows(32768, h, big, True, rows=rows, lib=lib)
        for x, i in enumerate(rows):
            assert int(mlt[x].sum()) == longnet_row_count(32768, big, h, i, True)


def pin_longnet_worked_example(lib):
    with open(os.path.join(GOLDEN, "longnet_sparsify_w16_r4.txt")) as f:
        lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(lines) >= 5
    for ln in lines:
        N, w, r, head, seg = map(int, ln[:5])
        kept = [int(x) for x in ln[5:]]
        mlt = oracle.longnet_mult_rows(N, head, [(w, r)], False, lib=lib)
        for i in range(seg * w, seg * w + w):
            keys = np.nonzero(mlt[i])[0].tolist()
            assert keys == (kept if i in kept else []), (ln, i)


def pin_longnet_offsets_partition(lib):
    # Across heads 0..r-1 every position of every segment is kept exactly once.
    for (N, w, r) in ((64, 16, 4), (100, 24, 6), (50, 50, 12)):
        cover = np.zeros(N, dtype=np.int64)
        for h in range(r):
            mlt = oracle.longnet_mult_rows(N, h, [(w, r)], True, lib=lib)
            cover += np.diag(mlt)
        assert (cover == 1).all()


def pin_dense_special_cases(lib):
    rng = np.random.default_rng(5)
    q, k, v = rand_qkv(rng, 2, 3, 37, 16)
    o_ref, l_ref = sdpa(q, k, v)
    oc_ref, lc_ref = sdpa(q, k, v, causal=True)
    # A window that covers the sequence is full attention (ETC lifting; Longformer).
    for R in (36, 100):
        o, l = oracle.attn_rows(q, k, v, (), R, lib=lib)
        assert np.abs(o - o_ref).max() < 1e-12 and np.abs(l - l_ref).max() < 1e-12
        o, l = oracle.attn_rows(q, k, v, (), R, None, True, lib=lib)
        assert np.abs(o - oc_ref).max() < 1e-12 and np.abs(l - lc_ref).max() < 1e-12
    # Every position global is full attention too.
    o, l = oracle.attn_rows(q, k, v, range(37), 0, lib=lib)
    assert np.abs(o - o_ref).max() < 1e-12
    # One LongNet pattern with w = N, r = 1 is dense (causal) attention.
    for causal, (orf, lrf) in ((True, (oc_ref, lc_ref)), (False, (o_ref, l_ref))):
        for fn in (oracle.longnet_rows, oracle.longnet_mixture_rows):
            o, l = fn(q, k, v, [(37, 1)], causal, lib=lib)
            assert np.abs(o - orf).max() < 1e-12 and np.abs(l - lrf).max() < 1e-12


def pin_global_rows_are_full_rows(lib):
    rng = np.random.default_rng(6)
    q, k, v = rand_qkv(rng, 1, 2, 45, 8)
    qg, kg, vg = rand_qkv(rng, 1, 2, 45, 8)
    G = (0, 3, 17, 44)
    o, l = oracle.attn_rows(q, k, v, G, 2, lib=lib)
    o_ref, l_ref = sdpa(q, k, v)
    assert np.abs(o[:, :, G] - o_ref[:, :, G]).max() < 1e-12
    o, l = oracle.attn_rows(q, k, v, G, 2, qg=qg, kg=kg, vg=vg, lib=lib)
    og_ref, lg_ref = sdpa(qg, kg, vg)
    assert np.abs(o[:, :, G] - og_ref[:, :, G]).max() < 1e-12
    assert np.abs(l[:, :, G] - lg_ref[:, :, G]).max() < 1e-12
    o2, _ = oracle.attn_rows(q, k, v, G, 2, lib=lib)  # non-global rows ignore qg, kg, vg
    ng = [i for i in range(45) if i not in G]
    assert np.abs(o[:, :, ng] - o2[:, :, ng]).max() < 1e-15


def pin_brute_force_band(lib):
    rnd = random.Random(3)
    rng = np.random.default_rng(3)
    for t in range(14):
        N = rnd.randint(1, 22)
        H = 2
        D = 4
        R = rnd.randint(0, 6)
        dil = [rnd.randint(1, 3) for _ in range(H)]
        causal = t % 2 == 1
        G = sorted(rnd.sample(range(N), rnd.randint(0, min(3, N))))
        sep = t % 3 == 0
        q, k, v = rand_qkv(rng, 1, H, N, D)
        qg, kg, vg = rand_qkv(rng, 1, H, N, D) if sep else (None, None, None)
        relb = rng.standard_normal((H, 7)) if t % 4 == 2 else None
        relv = rng.standard_normal((H, 7, D)) if t % 4 in (1, 2) else None
        seg = np.sort(rng.integers(0, 3, size=N)) if t % 5 in (0, 3) else None
        if t == 8:
            seg = rng.integers(0, 2, size=N)  # interleaved ids, not runs
        o, l = oracle.attn_rows(q, k, v, G, R, dil, causal, relb, qg, kg, vg, lib=lib,
                                rel_vec=relv, seg=None if seg is None else seg[None])
        for h in range(H):
            ob, lb = bf_band_head(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(), G, R,
                                  dil[h], causal,
                                  *(x[0, h].tolist() for x in (qg, kg, vg)) if sep else (None,) * 3,
                                  relb=None if relb is None else relb[h].tolist(),
                                  relv=None if relv is None else relv[h].tolist(),
                                  seg=None if seg is None else seg.tolist())
            assert np.abs(o[0, h] - ob).max() < 1e-12, (t, h)
            assert np.abs(l[0, h] - lb).max() < 1e-12, (t, h)


def pin_etc_four_pieces(lib):
    rng = np.random.default_rng(8)
    ng, nl, D, r = 5, 23, 4, 3
    for _ in range(3):
        xg = [rng.standard_normal((ng, D)) for _ in range(3)]
        xl = [rng.standard_normal((nl, D)) for _ in range(3)]
        relb = rng.standard_normal(2 * 2 + 1)
        ob, lb = bf_etc_four_pieces(*(x.tolist() for x in xg), *(x.tolist() for x in xl), r,
                                    relb.tolist())
        cat = [np.concatenate([a, b])[None, None] for a, b in zip(xg, xl)]
        o, l = oracle.attn_rows(*cat, range(ng), r, rel_bias=relb[None], lib=lib)
        assert np.abs(o[0, 0] - ob).max() < 1e-12
        assert np.abs(l[0, 0] - lb).max() < 1e-12


def pin_relvec_reduces_to_scalar(lib):
    """With every query's component 0 equal to sqrt(D) and a_l = b_l e_0, the
    vector term q_i . a_l / sqrt(D) is exactly the scalar b_l: the vector path
    must then equal the (separately pinned) scalar-table path. Separate global
    projections and causal windows included."""
    rng = np.random.default_rng(12)
    B, H, N, D, k = 1, 3, 37, 4, 5
    for t in range(4):
        q, kk, v = rand_qkv(rng, B, H, N, D)
        qg, kg, vg = rand_qkv(rng, B, H, N, D) if t % 2 else (None, None, None)
        q[..., 0] = math.sqrt(D)
        if qg is not None:
            qg[..., 0] = math.sqrt(D)
        b = rng.standard_normal((H, 2 * k + 1))
        a = np.zeros((H, 2 * k + 1, D))
        a[..., 0] = b
        G, R, causal = (0, 3, 17, 36), 4, t >= 2
        o1, l1 = oracle.attn_rows(q, kk, v, G, R, [1, 2, 1], causal, b, qg, kg, vg, lib=lib)
        o2, l2 = oracle.attn_rows(q, kk, v, G, R, [1, 2, 1], causal, None, qg, kg, vg, lib=lib,
                                  rel_vec=a)
        assert np.abs(o1 - o2).max() < 1e-12, t
        assert np.abs(l1 - l2).max() < 1e-12, t
        # both together add up: scalar b plus the vector's b again gives 2b
        o3, l3 = oracle.attn_rows(q, kk, v, G, R, [1, 2, 1], causal, b, qg, kg, vg, lib=lib,
                                  rel_vec=a)
        o4, l4 = oracle.attn_rows(q, kk, v, G, R, [1, 2, 1], causal, 2 * b, qg, kg, vg, lib=lib)
        assert np.abs(o3 - o4).max() < 1e-12, t
        assert np.abs(l3 - l4).max() < 1e-12, t


def pin_packing_equals_separate_documents(lib):
    """Documents packed into one input with segment masks (ETC page, §3.4
    "Per-instance attention masks") attend exactly as each document alone: the
    window, global rows and columns, dilation, causality, separate
    projections and relative labels all stay inside a document."""
    rng = np.random.default_rng(13)
    H, D = 2, 4
    # per batch row: document lengths and each document's local global tokens
    layouts = [[(9, (0, 1)), (14, (2,)), (6, ()), (11, (0, 10))],
               [(17, (3, 4)), (23, (0,))]]
    N = max(sum(n for n, _ in lay) for lay in layouts)
    for causal, R, dil, sep, rel in ((False, 3, [1, 2], False, True), (True, 4, [2, 1], True, False)):
        B = len(layouts)
        q, k, v = rand_qkv(rng, B, H, N, D)
        qg, kg, vg = rand_qkv(rng, B, H, N, D) if sep else (None, None, None)
        relb = rng.standard_normal((H, 7)) if rel else None
        relv = rng.standard_normal((H, 7, D)) if rel else None
        for b, lay in enumerate(layouts):
            seg = np.full(N, len(lay), dtype=np.int32)  # the tail past the last document
            G, off = [], 0
            for dn, (n, gl) in enumerate(lay):
                seg[off:off + n] = dn
                G += [off + g for g in gl]
                off += n
            # the packed row b alone as a batch of one (global positions differ per row)
            one = lambda x: None if x is None else x[b:b + 1]
            o, l = oracle.attn_rows(one(q), one(k), one(v), G, R, dil, causal, relb, one(qg), one(kg),
                                    one(vg), lib=lib, rel_vec=relv, seg=seg[None])
            off = 0
            for n, gl in lay:
                part = lambda x: None if x is None else x[b:b + 1, :, off:off + n]
                od, ld = oracle.attn_rows(part(q), part(k), part(v), gl, R, dil, causal, relb,
                                          part(qg), part(kg), part(vg), lib=lib, rel_vec=relv)
                assert np.abs(o[0, :, off:off + n] - od[0]).max() < 1e-12, (b, off)
                assert np.abs(l[0, :, off:off + n] - ld[0]).max() < 1e-12, (b, off)
                off += n
    # each batch row takes its own segment ids: two rows with different
    # segmentations in one call equal the rows called alone
    B, N = 2, 30
    q, k, v = rand_qkv(rng, B, H, N, D)
    segs = np.stack([np.repeat([0, 1, 2], [7, 12, 11]), np.repeat([0, 1], [20, 10])]).astype(np.int32)
    G = (0, 9, 25)
    o, l = oracle.attn_rows(q, k, v, G, 3, None, False, lib=lib, seg=segs)
    for b in range(B):
        ob, lb = oracle.attn_rows(q[b:b + 1], k[b:b + 1], v[b:b + 1], G, 3, None, False, lib=lib,
                                  seg=segs[b:b + 1])
        assert np.abs(o[b] - ob[0]).max() < 1e-12, b
        assert np.abs(l[b] - lb[0]).max() < 1e-12, b


def _fixed_keys(i, N, h, l, c, causal):
    """Sparse Transformer fixed pattern by enumeration: the query's own block,
    plus offsets l - c(h'+1) .. l - c h' - 1 of every block, h' = h mod (l // c)."""
    hp = h % max(1, l // c)
    run = set(range(l - c * (hp + 1), l - c * hp))
    keys = {j for j in range(N) if j // l == i // l} | {j for j in range(N) if j % l in run}
    return sorted(j for j in keys if not causal or j <= i)


def pin_fixed_pattern(lib):
    """Fixed pattern: brute force on tiny inputs; c = l (every position a
    summary) is dense attention; key counts in closed form; the heads' summary
    runs tile the block."""
    rng = np.random.default_rng(14)
    for (N, l, c, causal) in ((40, 8, 2, True), (36, 12, 4, False), (30, 10, 3, True)):
        H, D = 4, 4
        q, k, v = rand_qkv(rng, 1, H, N, D)
        o, lse = oracle.fixed_rows(q, k, v, l, c, causal, lib=lib)
        for h in range(H):
            for i in range(N):
                ob, lb = bf_attend(q[0, h, i].tolist(), _fixed_keys(i, N, h, l, c, causal),
                                   k[0, h].tolist(), v[0, h].tolist())
                assert np.abs(o[0, h, i] - ob).max() < 1e-12, (N, l, c, h, i)
                assert abs(lse[0, h, i] - lb) < 1e-12
    q, k, v = rand_qkv(rng, 2, 3, 37, 16)
    for causal in (True, False):
        o_ref, l_ref = sdpa(q, k, v, causal=causal)
        o, l = oracle.fixed_rows(q, k, v, 8, 8, causal, lib=lib)
        assert np.abs(o - o_ref).max() < 1e-12 and np.abs(l - l_ref).max() < 1e-12
    # counts through exp(lse) with q = 0: causal row i in block b at offset o
    # sees o + 1 keys of its block and c of each earlier block; non-causal, the
    # whole block and c of every other block
    N, l, c, H = 96, 16, 4, 4
    z = np.zeros((1, H, N, 8))
    for causal in (True, False):
        _, lse = oracle.fixed_rows(z, z, z, l, c, causal, lib=lib)
        i = np.arange(N)
        want = (i % l + 1 + (i // l) * c) if causal else (l + (N // l - 1) * c) * np.ones(N)
        assert np.array_equal(np.rint(np.exp(lse[0])).astype(np.int64),
                              np.broadcast_to(want, (H, N)).astype(np.int64)), causal
    # the l // c heads' summary runs partition the block offsets
    seen = sorted(o for h in range(l // c) for o in range(l) if
                  o in range(l - c * (h % (l // c) + 1), l - c * (h % (l // c))))
    assert seen == list(range(l))


def pin_brute_force_longnet(lib):
    rng = np.random.default_rng(9)
    cases = [(24, ((4, 1), (8, 2), (24, 4)), True), (21, ((6, 1), (12, 3)), True),
             (20, ((8, 2), (20, 5)), False), (16, ((16, 4),), True)]
    for N, pairs, causal in cases:
        H, D = 6, 4
        q, k, v = [x * 0.5 for x in rand_qkv(rng, 1, H, N, D)]
        o1, l1 = oracle.longnet_rows(q, k, v, pairs, causal, lib=lib)
        o2, l2 = oracle.longnet_mixture_rows(q, k, v, pairs, causal, lib=lib)
        for h in range(H):
            ob, lb = bf_longnet_head(q[0, h].tolist(), k[0, h].tolist(), v[0, h].tolist(),
                                     pairs, h, causal)
            fin = np.isfinite(lb)
            for o, l in ((o1, l1), (o2, l2)):
                assert np.abs(o[0, h] - ob).max() < 1e-12, (N, pairs, h)
                assert np.array_equal(np.isfinite(l[0, h]), fin)
                assert np.abs(l[0, h][fin] - lb[fin]).max() < 1e-12


def pin_longnet_paths_agree(lib):
    rng = np.random.default_rng(10)
    pairs = ((32, 1), (64, 2), (128, 4), (192, 6), (200, 12))
    q, k, v = rand_qkv(rng, 1, 12, 200, 16)
    for causal in (True, False):
        o1, l1 = oracle.longnet_rows(q, k, v, pairs, causal, lib=lib)
        o2, l2 = oracle.longnet_mixture_rows(q, k, v, pairs, causal, lib=lib)
        assert np.abs(o1 - o2).max() < 1e-12 and np.abs(l1 - l2).max() < 1e-12
    # A pattern listed twice changes no output; lse rises by ln 2.
    o3, l3 = oracle.longnet_rows(q, k, v, pairs[:2] + pairs[:2], True, lib=lib)
    o4, l4 = oracle.longnet_rows(q, k, v, pairs[:2], True, lib=lib)
    assert np.abs(o3 - o4).max() < 1e-12 and np.abs(l3 - l4 - math.log(2)).max() < 1e-12
    o5, _ = oracle.longnet_mixture_rows(q, k, v, pairs[:2] + pairs[:2], True, lib=lib)
    assert np.abs(o5 - o4).max() < 1e-12


def pin_rows_sum_to_one(lib):
    rng = np.random.default_rng(12)
    q, k, _ = rand_qkv(rng, 1, 2, 60, 8)
    ones = np.ones_like(q)
    o, _ = oracle.attn_rows(q, k, ones, (1, 30), 5, [1, 3], True, lib=lib)
    assert np.abs(o - 1).max() < 1e-13
    o, _ = oracle.longnet_rows(q, k, ones, ((8, 1), (16, 2)), True, lib=lib)
    assert np.abs(o - 1).max() < 1e-13


def pin_uncovered_rows(lib):
    # A single r=2 pattern leaves odd rows of head 0 uncovered: O = 0, lse = -inf.
    rng = np.random.default_rng(13)
    q, k, v = rand_qkv(rng, 1, 2, 16, 4)
    for fn in (oracle.longnet_rows, oracle.longnet_mixture_rows):
        o, l = fn(q, k, v, [(8, 2)], True, lib=lib)
        assert np.isneginf(l[0, 0, 1::2]).all() and (o[0, 0, 1::2] == 0).all()
        assert np.isfinite(l[0, 0, 0::2]).all() and np.isfinite(l[0, 1, 1::2]).all()


def pin_sampled_rows_match_full(lib):
    rng = np.random.default_rng(14)
    q, k, v = rand_qkv(rng, 2, 3, 50, 8)
    o, l = oracle.attn_rows(q, k, v, (4,), 3, [1, 2, 1], True, lib=lib)
    sel = np.array([[1, 2, 49], [0, 0, 0], [1, 1, 4], [0, 1, 17]])
    os_, ls_ = oracle.attn_rows(q, k, v, (4,), 3, [1, 2, 1], True, sel=sel, lib=lib)
    for x, (b, h, i) in enumerate(sel):
        assert np.array_equal(os_[x], o[b, h, i]) and ls_[x] == l[b, h, i]


# --- backward -------------------------------------------------------------

def _fd_loss(lib, args, kw, dout):
    o, _ = oracle.attn_rows(*args, **kw, lib=lib)
    return float((o * dout).sum())


def pin_backward_finite_differences(lib):
    """The backward against central differences of the forward's loss sum(dO * O)
    (fp64, eps 1e-6): shared and separate projections, causal, dilation, segments."""
    cases = [
        dict(N=16, glob=(0, 5), R=2, dil=[1, 2], causal=False, sep=False, seg=False),
        dict(N=18, glob=(3, 11), R=3, dil=[2, 1], causal=True, sep=True, seg=False),
        dict(N=16, glob=(0, 8), R=2, dil=[1, 1], causal=False, sep=True, seg=True),
    ]
    rng = np.random.default_rng(21)
    for c in cases:
        B, H, N, D = 2, 2, c["N"], 4
        q, k, v = rand_qkv(rng, B, H, N, D)
        qg, kg, vg = rand_qkv(rng, B, H, N, D) if c["sep"] else (None, None, None)
        seg = np.repeat(np.arange(2), N // 2)[None].repeat(B, 0) if c["seg"] else None
        dout = rng.standard_normal((B, H, N, D))
        grads = oracle.attn_backward(q, k, v, dout, c["glob"], c["R"], c["dil"], c["causal"],
                                     qg, kg, vg, seg=seg, lib=lib)
        tensors = [q, k, v] + ([qg, kg, vg] if c["sep"] else [])
        kw = dict(global_idx=c["glob"], radius=c["R"], dilation=c["dil"], causal=c["causal"],
                  qg=qg, kg=kg, vg=vg, seg=seg)
        eps = 1e-6
        for t, g in zip(tensors, grads):
            coords = [tuple(rng.integers(0, n) for n in t.shape) for _ in range(6)]
            coords += [(0, 1, c["glob"][0], 2), (1, 0, c["glob"][1], 0)]  # global rows / keys
            for x in coords:
                old = t[x]
                t[x] = old + eps
                lp = _fd_loss(lib, (q, k, v), kw, dout)
                t[x] = old - eps
                lm = _fd_loss(lib, (q, k, v), kw, dout)
                t[x] = old
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - g[x]) <= 1e-6 * (1 + abs(fd)), (c, x, fd, g[x])


def pin_backward_labels_finite_differences(lib):
    """The backward with a scalar bias table, key-side label vectors, per-pair
    label matrices (masked pairs among them) and segment masks on some pieces,
    against central differences of the forward's loss sum(dO * O) (fp64, eps
    1e-6); the tables are inputs, not differentiated."""
    rng = np.random.default_rng(29)
    cases = [
        dict(N=17, glob=(0, 6, 7), R=2, dil=[1, 2], causal=False, sep=True, pieces=9, kk=2, ns=3),
        dict(N=15, glob=(2, 9), R=3, dil=[1, 1], causal=True, sep=False, pieces=6, kk=1, ns=2),
    ]
    for c in cases:
        B, H, N, D = 2, 2, c["N"], 4
        G = c["glob"]
        V = 2 * c["kk"] + 1 + c["ns"]
        q, k, v = rand_qkv(rng, B, H, N, D)
        qg, kg, vg = rand_qkv(rng, B, H, N, D) if c["sep"] else (None, None, None)
        tab = 0.5 * rng.standard_normal((H, V))
        vec = 0.5 * rng.standard_normal((H, V, D))
        vals = [0, 1, V - 1, DIST, DIST, DIST, MASK]
        glabel = rng.choice(vals, size=(B, len(G), N)).astype(np.uint8)
        llabel = rng.choice(vals, size=(B, N, len(G))).astype(np.uint8)
        seg = (np.arange(N)[None] * 3 // N).repeat(B, 0)
        dout = rng.standard_normal((B, H, N, D))
        kw = dict(global_idx=G, radius=c["R"], dilation=c["dil"], causal=c["causal"], qg=qg,
                  kg=kg, vg=vg, seg=seg, rel_bias=tab, rel_vec=vec, rel_k=c["kk"],
                  glabel=glabel, llabel=llabel, seg_pieces=c["pieces"])
        grads = oracle.attn_backward(q, k, v, dout, lib=lib, **kw)
        tensors = [q, k, v] + ([qg, kg, vg] if c["sep"] else [])
        eps = 1e-6
        for t, g in zip(tensors, grads):
            coords = [tuple(rng.integers(0, n) for n in t.shape) for _ in range(8)]
            coords += [(0, 1, G[0], 2), (1, 0, G[1], 0)]  # global rows / keys
            for x in coords:
                old = t[x]
                t[x] = old + eps
                lp = _fd_loss(lib, (q, k, v), kw, dout)
                t[x] = old - eps
                lm = _fd_loss(lib, (q, k, v), kw, dout)
                t[x] = old
                fd = (lp - lm) / (2 * eps)
                assert abs(fd - g[x]) <= 1e-6 * (1 + abs(fd)), (c, x, fd, g[x])


def pin_backward_dense_autograd(lib):
    """A window covering every key, no global token: the gradients of dense
    softmax attention, from torch autograd in float64."""
    rng = np.random.default_rng(22)
    for causal in (False, True):
        q, k, v = rand_qkv(rng, 1, 2, 12, 8)
        dout = rng.standard_normal(q.shape)
        grads = oracle.attn_backward(q, k, v, dout, (), 12, None, causal, lib=lib)
        t = [torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v)]
        s = t[0] @ t[1].transpose(-1, -2) / math.sqrt(8)
        if causal:
            s = s.masked_fill(torch.ones(12, 12, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.softmax(s, -1) @ t[2]
        o.backward(torch.from_numpy(dout))
        for a, b in zip(grads, t):
            assert np.allclose(a, b.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_backward_shift_invariants(lib):
    """Shifting every key of one projection by c moves each row's logits by a
    constant, so the keys' gradients sum to 0; shifting every value by c moves
    each output by c, so the values' gradients sum to the rows' dO (per head,
    per projection set)."""
    rng = np.random.default_rng(23)
    B, H, N, D = 1, 3, 40, 6
    q, k, v = rand_qkv(rng, B, H, N, D)
    qg, kg, vg = rand_qkv(rng, B, H, N, D)
    dout = rng.standard_normal(q.shape)
    glob = (2, 17, 30)
    dq, dk, dv, dqg, dkg, dvg = oracle.attn_backward(q, k, v, dout, glob, 4, [1, 3, 2], True,
                                                     qg, kg, vg, lib=lib)
    isg = np.zeros(N, bool)
    isg[list(glob)] = True
    assert np.allclose(dk.sum(2), 0, atol=1e-12) and np.allclose(dkg.sum(2), 0, atol=1e-12)
    assert np.allclose(dv.sum(2), dout[:, :, ~isg].sum(2), atol=1e-12)
    assert np.allclose(dvg.sum(2), dout[:, :, isg].sum(2), atol=1e-12)
    # global rows touch only the separate projections' gradients, and conversely
    assert (dqg[:, :, ~isg] == 0).all() and (dq[:, :, isg] == 0).all()


def pin_longnet_backward(lib):
    """The LongNet mixture's backward against central differences of its forward
    loss (overlapping patterns, so some keys count twice); a single (N, 1)
    pattern against torch float64 autograd of dense causal attention; the
    keys' gradients summing to 0 per head."""
    rng = np.random.default_rng(24)
    B, H, N, D = 1, 3, 24, 4
    q, k, v = rand_qkv(rng, B, H, N, D)
    dout = rng.standard_normal(q.shape)
    pairs = [(8, 1), (16, 2), (24, 3)]
    for causal in (True, False):
        dq, dk, dv = oracle.longnet_backward(q, k, v, dout, pairs, causal, lib=lib)
        assert np.allclose(dk.sum(2), 0, atol=1e-12)
        for t, g in ((q, dq), (k, dk), (v, dv)):
            for _ in range(6):
                x = tuple(rng.integers(0, n) for n in t.shape)
                old = t[x]
                t[x] = old + 1e-6
                lp = float((oracle.longnet_rows(q, k, v, pairs, causal, lib=lib)[0] * dout).sum())
                t[x] = old - 1e-6
                lm = float((oracle.longnet_rows(q, k, v, pairs, causal, lib=lib)[0] * dout).sum())
                t[x] = old
                fd = (lp - lm) / 2e-6
                assert abs(fd - g[x]) <= 1e-6 * (1 + abs(fd)), (causal, x, fd, g[x])
    q, k, v = rand_qkv(rng, 1, 2, 16, 8)
    dout = rng.standard_normal(q.shape)
    grads = oracle.longnet_backward(q, k, v, dout, [(16, 1)], True, lib=lib)
    t = [torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v)]
    sc = (t[0] @ t[1].transpose(-1, -2) / math.sqrt(8)).masked_fill(
        torch.ones(16, 16, dtype=torch.bool).triu(1), float("-inf"))
    (torch.softmax(sc, -1) @ t[2]).backward(torch.from_numpy(dout))
    for a_, b_ in zip(grads, t):
        assert np.allclose(a_, b_.grad.numpy(), rtol=1e-10, atol=1e-12)


def pin_longnet_per_pattern_outputs(lib):
    """The page-order mixture's per-pattern outputs: pattern k's O_k and lse_k
    equal the mixture of that single pattern alone (for a row the pattern skips,
    O_k = 0 and lse_k = -inf), and mixing them with weights e^{lse_k} gives the
    mixture's own output."""
    rng = np.random.default_rng(25)
    pairs = ((8, 1), (16, 2), (24, 3), (20, 4))
    q, k, v = rand_qkv(rng, 2, 5, 40, 6)
    for causal in (True, False):
        o, l, ok, lk = oracle.longnet_mixture_rows(q, k, v, pairs, causal, per_pattern=True,
                                                   lib=lib)
        ok, lk = ok.reshape(len(pairs), -1, 6), lk.reshape(len(pairs), -1)
        for p_, pair in enumerate(pairs):
            o1, l1 = oracle.longnet_rows(q, k, v, [pair], causal, lib=lib)
            fin = np.isfinite(l1.reshape(-1))
            assert np.array_equal(np.isfinite(lk[p_]), fin), (pair, causal)
            assert np.abs(lk[p_][fin] - l1.reshape(-1)[fin]).max() < 1e-12
            assert np.abs(ok[p_] - o1.reshape(-1, 6)).max() < 1e-12
            assert (ok[p_][~fin] == 0).all()
        wgt = np.exp(lk - l.reshape(-1)[None])
        assert np.abs((wgt[..., None] * ok).sum(0) - o.reshape(-1, 6)).max() < 1e-12


def pin_longnet_backward_selected(lib):
    """Chosen-row / chosen-key gradients against the full backward (itself
    pinned by finite differences), with overlapping patterns so that some
    pairs count twice, rows no pattern covers, and a ragged last segment."""
    rng = np.random.default_rng(26)
    B, H, N, D = 2, 4, 30, 4
    q, k, v = rand_qkv(rng, B, H, N, D)
    dout = rng.standard_normal(q.shape)
    for pairs, causal in ((((8, 1), (16, 2), (16, 1), (30, 4)), True),
                          (((12, 2), (30, 3)), False)):
        dq, dk, dv = oracle.longnet_backward(q, k, v, dout, pairs, causal, lib=lib)
        allr = np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(N)])
        sq, sk, sv = oracle.longnet_backward_sel(q, k, v, dout, pairs, causal, rows=allr,
                                                 keys=allr[::-1], lib=lib)
        assert np.abs(sq - dq.reshape(-1, D)).max() < 1e-12, pairs
        assert np.abs(sk[::-1] - dk.reshape(-1, D)).max() < 1e-12, pairs
        assert np.abs(sv[::-1] - dv.reshape(-1, D)).max() < 1e-12, pairs


DIST, MASK = oracle.LABEL_DISTANCE, oracle.LABEL_MASKED


def bf_etc_structured(qg_, kg_, vg_, ql, kl, vl, r, tab, vec, M, L, kk):
    """ETC global-local attention from its four pieces with explicit per-piece
    masks M[piece] (1 = edge) and per-pair labels L[piece] (a vocabulary index,
    or None for the clipped-distance label); the logit of an edge with label l
    is q_i . (k_j + a_l) / sqrt(D) + b_l. l2l also needs |i - j| <= r."""
    ng, nl = len(qg_), len(ql)
    D = len(ql[0])
    sc = 1.0 / math.sqrt(D)

    def logit(qi, kj, lab):
        e = sc * _dot(qi, kj)
        if lab is not None:
            e += tab[lab] + sc * _dot(qi, vec[lab])
        return e

    def dist(i, j):
        return max(-kk, min(kk, j - i)) + kk

    out, lse = [], []
    for i in range(ng):  # one softmax over [g2g ; g2l]
        e, vals = [], []
        for j in range(ng):
            if M["g2g"][i][j]:
                lab = L["g2g"][i][j]
                e.append(logit(qg_[i], kg_[j], dist(i, j) if lab is None else lab))
                vals.append(vg_[j])
        for j in range(nl):
            if M["g2l"][i][j]:
                e.append(logit(qg_[i], kl[j], L["g2l"][i][j]))
                vals.append(vl[j])
        out_i, lse_i = _softmax_mix(e, vals, D)
        out.append(out_i)
        lse.append(lse_i)
    for i in range(nl):  # one softmax over [l2g ; l2l]
        e, vals = [], []
        for j in range(ng):
            if M["l2g"][i][j]:
                e.append(logit(ql[i], kg_[j], L["l2g"][i][j]))
                vals.append(vg_[j])
        for j in range(max(0, i - r), min(nl, i + r + 1)):
            if M["l2l"][i][j]:
                e.append(logit(ql[i], kl[j], dist(i, j)))
                vals.append(vl[j])
        out_i, lse_i = _softmax_mix(e, vals, D)
        out.append(out_i)
        lse.append(lse_i)
    return np.array(out), np.array(lse)


def _softmax_mix(e, vals, D):
    if not e:
        return [0.0] * D, -math.inf
    Mx = max(e)
    p = [math.exp(x - Mx) for x in e]
    Z = sum(p)
    return [sum(p[t] * vals[t][c] for t in range(len(p))) / Z for c in range(D)], Mx + math.log(Z)


def pin_etc_structured_pieces(lib):
    """Per-instance per-piece masks and structural labels (ETC page, 3.4
    "Per-instance attention masks", "How Global-Local Attention Encodes
    Structured Inputs", "Relative Position Encoding" Step 1): two contexts of
    two sentences each; global input = CLS, one token per context, one per
    sentence, one candidate answer; hard g2l (a sentence token sees only its
    sentence's word pieces), no cross-context g2g for sentence tokens (context
    tokens exempt), no cross-context l2l; labels belongs / does-not-belong on
    sentence <-> word-piece edges, mention on candidate <-> mention edges,
    part-of on sentence -> context edges. The four-piece brute force with the
    explicit matrices equals the oracle's one concatenated call."""
    rng = np.random.default_rng(27)
    D, kk, r = 4, 2, 2
    sent = [0] * 4 + [1] * 3 + [2] * 5 + [3] * 4   # word piece -> sentence
    ctx_of_sent = [0, 0, 1, 1]
    nl = len(sent)
    ctx = [ctx_of_sent[s_] for s_ in sent]
    # global tokens: 0 CLS, 1-2 contexts, 3-6 sentences, 7 candidate
    kind = ["cls", "ctx", "ctx", "sent", "sent", "sent", "sent", "cand"]
    gctx = [None, 0, 1, 0, 0, 1, 1, None]
    gsent = [None, None, None, 0, 1, 2, 3, None]
    mention = {5, 12}          # word pieces mentioning the candidate
    ng = len(kind)
    V = 2 * kk + 1 + 4
    BEL, NOT, MEN, PART = 2 * kk + 1, 2 * kk + 2, 2 * kk + 3, 2 * kk + 4
    M = {p_: [[1] * (ng if p_.endswith("2g") else nl) for _ in range(ng if p_[0] == "g" else nl)]
         for p_ in ("g2g", "g2l", "l2g", "l2l")}
    L = {p_: [[None] * (ng if p_.endswith("2g") else nl) for _ in range(ng if p_[0] == "g" else nl)]
         for p_ in ("g2g", "g2l", "l2g")}
    for g in range(ng):
        for j in range(nl):
            if kind[g] == "sent":
                M["g2l"][g][j] = int(sent[j] == gsent[g])            # hard g2l
                L["g2l"][g][j] = BEL if sent[j] == gsent[g] else NOT
            if kind[g] == "cand" and j in mention:
                L["g2l"][g][j] = MEN
        for g2 in range(ng):
            if kind[g] == "sent" and kind[g2] == "sent" and gctx[g] != gctx[g2]:
                M["g2g"][g][g2] = 0                                 # cross-context sentence pair
            if kind[g] == "sent" and kind[g2] == "ctx" and gctx[g] == gctx[g2]:
                L["g2g"][g][g2] = PART
    for i in range(nl):
        for g in range(ng):
            if kind[g] == "sent":
                L["l2g"][i][g] = BEL if sent[i] == gsent[g] else NOT
            if kind[g] == "cand" and i in mention:
                L["l2g"][i][g] = MEN
        for j in range(nl):
            M["l2l"][i][j] = int(ctx[i] == ctx[j])                   # no cross-context l2l
    q = rng.standard_normal((1, 2, ng + nl, D))
    k = rng.standard_normal((1, 2, ng + nl, D))
    v = rng.standard_normal((1, 2, ng + nl, D))
    tab = 0.3 * rng.standard_normal((2, V))
    vec = 0.3 * rng.standard_normal((2, V, D))
    N = ng + nl
    glabel = np.full((1, ng, N), DIST, dtype=np.uint8)
    llabel = np.full((1, N, ng), DIST, dtype=np.uint8)
    for g in range(ng):
        for j in range(N):
            piece, jj = ("g2g", j) if j < ng else ("g2l", j - ng)
            lab = L[piece][g][jj]
            glabel[0, g, j] = MASK if not M[piece][g][jj] else (DIST if lab is None else lab)
    for i in range(nl):
        for g in range(ng):
            lab = L["l2g"][i][g]
            llabel[0, ng + i, g] = MASK if not M["l2g"][i][g] else (DIST if lab is None else lab)
    seg = np.array([[0] * ng + [c_ + 1 for c_ in ctx]])  # l2l only
    o, l = oracle.attn_rows(q, k, v, range(ng), r, rel_bias=tab, rel_vec=vec, rel_k=kk,
                            glabel=glabel, llabel=llabel, seg=seg, seg_pieces=8, lib=lib)
    for h in range(2):
        ob, lb = bf_etc_structured(q[0, h, :ng].tolist(), k[0, h, :ng].tolist(),
                                   v[0, h, :ng].tolist(), q[0, h, ng:].tolist(),
                                   k[0, h, ng:].tolist(), v[0, h, ng:].tolist(), r, tab[h],
                                   vec[h].tolist(), M, L, kk)
        assert np.abs(o[0, h] - ob).max() < 1e-12, h
        assert np.abs(l[0, h] - lb).max() < 1e-12, h


def pin_labels_scattered_globals(lib):
    """Label inputs with scattered global positions (Longformer layout, a
    dilated head, separate global projections): against masked softmax over an
    explicit label matrix built position by position; and all-default labels
    equal no label input at all."""
    rng = np.random.default_rng(28)
    B, H, N, D, R, kk = 2, 2, 30, 4, 3, 2
    G = [2, 9, 10, 23]
    V = 2 * kk + 1 + 2
    q, k, v = rand_qkv(rng, B, H, N, D)
    qg, kg, vg = rand_qkv(rng, B, H, N, D)
    tab = 0.3 * rng.standard_normal((H, V))
    vec = 0.3 * rng.standard_normal((H, V, D))
    glabel = rng.choice([0, 3, V - 1, V - 2, DIST, DIST, MASK], size=(B, len(G), N)).astype(np.uint8)
    llabel = rng.choice([1, V - 1, DIST, MASK, 200], size=(B, N, len(G))).astype(np.uint8)
    dil = [1, 2]
    o, l = oracle.attn_rows(q, k, v, G, R, dil, False, tab, qg, kg, vg, rel_vec=vec, rel_k=kk,
                            glabel=glabel, llabel=llabel, lib=lib)
    sc = 1.0 / math.sqrt(D)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                ig = i in G
                Q, K_, V_ = (qg, kg, vg) if ig else (q, k, v)
                e, vals = [], []
                for j in range(N):
                    jg = j in G
                    band = (j - i) % dil[h] == 0 and abs(j - i) <= dil[h] * R
                    if not (ig or jg or band):
                        continue
                    if ig:
                        lab = int(glabel[b, G.index(i), j])
                    elif jg:
                        lab = int(llabel[b, i, G.index(j)])
                    else:
                        lab = DIST
                    if lab != DIST and lab >= V:
                        continue                       # masked pair
                    if lab == DIST:
                        lab = (max(-kk, min(kk, j - i)) + kk) if ig == jg else None
                    x = sc * _dot(Q[b, h, i], K_[b, h, j])
                    if lab is not None:
                        x += tab[h, lab] + sc * _dot(Q[b, h, i], vec[h, lab])
                    e.append(x)
                    vals.append(V_[b, h, j].tolist())
                ob, lb = _softmax_mix(e, vals, D)
                assert np.abs(o[b, h, i] - ob).max() < 1e-12, (b, h, i)
                assert (np.isneginf(lb) and np.isneginf(l[b, h, i])) or abs(l[b, h, i] - lb) < 1e-12
    dflt = np.full_like(glabel, DIST), np.full_like(llabel, DIST)
    o1, l1 = oracle.attn_rows(q, k, v, G, R, dil, False, tab[:, :2 * kk + 1], qg, kg, vg,
                              rel_vec=vec[:, :2 * kk + 1], glabel=dflt[0], llabel=dflt[1], lib=lib)
    o2, l2 = oracle.attn_rows(q, k, v, G, R, dil, False, tab[:, :2 * kk + 1], qg, kg, vg,
                              rel_vec=vec[:, :2 * kk + 1], lib=lib)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


PINS = [pin_mask_matches_enumeration, pin_counts_closed_form, pin_counts_full_workloads,
        pin_longnet_counts, pin_longnet_worked_example, pin_longnet_offsets_partition,
        pin_dense_special_cases, pin_global_rows_are_full_rows, pin_brute_force_band,
        pin_etc_four_pieces, pin_relvec_reduces_to_scalar, pin_packing_equals_separate_documents,
        pin_fixed_pattern, pin_brute_force_longnet,
        pin_longnet_paths_agree,
        pin_rows_sum_to_one, pin_uncovered_rows, pin_sampled_rows_match_full,
        pin_backward_finite_differences, pin_backward_labels_finite_differences,
        pin_backward_dense_autograd,
        pin_backward_shift_invariants, pin_longnet_backward, pin_longnet_per_pattern_outputs,
        pin_longnet_backward_selected, pin_etc_structured_pieces, pin_labels_scattered_globals]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.load())


# Plausible mistakes, planted in a copy of oracle.cpp: (name, original, replacement).
MUTANTS = [
    ("causal-direction", "const int64_t delta = (int64_t)j - (int64_t)i;",
     "const int64_t delta = (int64_t)i - (int64_t)j;"),
    ("exclusive-window-end", "return steps >= -(int64_t)radius && steps <= (int64_t)radius;",
     "return steps >= -(int64_t)radius && steps < (int64_t)radius;"),
    ("dropped-scale", "logit[j] = dot * scale + bias(j);", "logit[j] = dot + bias(j);"),
    ("bias-index-sign", "l = (int32_t)(dlt + rel_k);", "l = (int32_t)(rel_k - dlt);"),
    ("segments-ignored-by-global-rows", "if (sb && (pieces & piece) && sb[j] != sb[i]) weight[j] = 0.0;",
     "if (sb && (pieces & piece) && sb[j] != sb[i] && !ig) weight[j] = 0.0;"),
    ("segments-of-another-batch-row", "const int32_t* sb = seg ? seg + (size_t)b * N : nullptr;",
     "const int32_t* sb = seg ? seg : nullptr;"),
    ("fixed-one-subblock-for-all-heads", "const int32_t hp = head % std::max(1, l / c);",
     "const int32_t hp = 0;"),
    ("fixed-run-one-too-long", "return o >= t && o < t + c;", "return o >= t && o <= t + c;"),
    ("fixed-ignores-causal", "  if (causal && j > i) return false;\n  if (i / l == j / l) return true;",
     "  if (i / l == j / l) return true;"),
    ("relvec-label-sign", "const double* al = vec + (size_t)l * D;",
     "const double* al = vec + (size_t)(2 * rel_k - l) * D;"),
    ("relvec-unscaled", "b += dot * scale;", "b += dot;"),
    ("relvec-against-key", "for (int32_t d = 0; d < D; ++d) dot += qi[d] * al[d];",
     "for (int32_t d = 0; d < D; ++d) dot += kb[(size_t)j * D + d] * al[d];"),
    ("bias-on-mixed-pairs", "if (jg != ig) {", "if (false) {"),
    ("shared-keys-for-global-rows", "const double* kb = (sep ? kg : k) + head_off;",
     "const double* kb = (sep ? k : k) + head_off;"),
    ("keys-as-values", "const double* vj = vbase + (size_t)j * D;",
     "const double* vj = kbase + (size_t)j * D;"),
    ("lse-without-max", "*lse = M + std::log(Z);", "*lse = std::log(Z);"),
    ("global-ignores-causal", "  if (causal && j > i) return 0;\n  if (i_glob || j_glob) return 1;",
     "  if (i_glob || j_glob) return 1;"),
    ("no-head-offset", "return ((p - seg_start) % r) == (head % r);",
     "return ((p - seg_start) % r) == 0;"),
    ("no-segment-check", "if (i / w[k] != j / w[k]) continue;  // same segment", ""),
    ("equal-mixture-weights", "const double alpha = std::exp(Lk[p] - Lmax) / S;",
     "const double alpha = 1.0 / n_pairs;"),
    ("mixture-excludes-self", "if (!causal || j <= i) weight[j] = 1.0;",
     "if (!causal || j < i) weight[j] = 1.0;"),
    ("mixture-no-scatter", "if ((i - seg_start) % r[p] != off) continue;  // scattered zero row", ""),
    ("backward-without-delta", "const double dS = P[j] * (dP[j] - Di);",
     "const double dS = P[j] * dP[j];"),
    ("backward-dk-unscaled", "dkb[(size_t)j * D + d] += dS * qi[d] * scale;",
     "dkb[(size_t)j * D + d] += dS * qi[d];"),
    ("backward-dv-from-dS", "dvb[(size_t)j * D + d] += P[j] * doi[d];",
     "dvb[(size_t)j * D + d] += dS * doi[d];"),
    ("backward-global-keys-to-shared", "double* dkb = (sep ? dkg : dk) + off;",
     "double* dkb = dk + off;"),
    ("longnet-backward-multiplicity-one", "P[j] = c;  // the multiplicity for now",
     "P[j] = c ? 1 : 0;  // the multiplicity for now"),
    ("per-pattern-lse-is-mixture-lse", "lse_k[(size_t)p * rows + x] = Lk[p];",
     "lse_k[(size_t)p * rows + x] = Lmax;"),
    ("selected-delta-without-multiplicity",
     "row.Di += row.c[j] * std::exp(row.logit[j] - row.lse) * dp;",
     "row.Di += std::exp(row.logit[j] - row.lse) * dp;"),
    ("selected-dv-from-dS", "dvj[d] += P * doi[d];", "dvj[d] += g * doi[d];"),
    ("l2g-labels-transposed", "l = llabel[((size_t)b * N + i) * n_global + grank[j]];",
     "l = llabel[((size_t)b * n_global + grank[j]) * N + i];"),
    ("global-labels-by-position", "l = glabel[((size_t)b * n_global + grank[i]) * N + j];",
     "l = glabel[((size_t)b * n_global + i) * N + j];"),
    ("masked-label-ignored", "if (l != kLabelDistance && l >= V) weight[j] = 0.0;  // M = 0", ""),
    ("segments-mask-every-piece", "const int32_t pieces = seg_pieces ? seg_pieces : 15;",
     "const int32_t pieces = 15;"),
    ("explicit-labels-same-kind-only", "lab[j] = (has_tables && weight[j] != 0.0) ? l : -1;",
     "lab[j] = (has_tables && weight[j] != 0.0 && jg == ig) ? l : -1;"),
    ("backward-ignores-bias", "P[j] = dot * scale + (lab[j] >= 0 && tab ? tab[lab[j]] : 0.0);",
     "P[j] = dot * scale;"),
    ("backward-dq-without-label-vector",
     "dqi[d] += dS * (kb[(size_t)j * D + d] + (al ? al[d] : 0.0)) * scale;",
     "dqi[d] += dS * kb[(size_t)j * D + d] * scale;"),
    ("selected-dq-unscaled", "for (int32_t d = 0; d < D; ++d) dqi[d] += g * k[off + (size_t)j * D + d] * scale;",
     "for (int32_t d = 0; d < D; ++d) dqi[d] += g * k[off + (size_t)j * D + d];"),
]


def test_planted_mistakes_are_caught():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        missed = []
        for name, old, new in MUTANTS:
            assert src.count(old) == 1, f"mutation {name!r} does not match oracle.cpp exactly once"
            path = os.path.join(tmp, f"{name}.cpp")
            with open(path, "w") as f:
                f.write(src.replace(old, new))
            so = oracle.build(path, os.path.join(tmp, f"lib{name}.so"), strict=False)
            lib = oracle.load(so)
            caught = False
            for pin in PINS:
                try:
                    pin(lib)
                except (AssertionError, ValueError):
                    caught = True
                    break
            if not caught:
                missed.append(name)
        assert not missed, f"planted mistakes no pin catches: {missed}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
