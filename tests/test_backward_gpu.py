"""Parity of the HIP backward (la_attn_backward) with the fp64 oracle's backward.

The GPU forward supplies out and lse (the backward's inputs by contract); the
oracle gets only q, k, v (and qg, kg, vg), the mask arguments and dout, and
recomputes everything else in fp64.

Bar, element-wise: |gpu - oracle| <= a * max|oracle| + b * |oracle| for every
entry of every gradient tensor, with (a, b) = (2e-6, 2e-5) for fp32 inputs and
(5e-3, 1e-2) for bf16. For bf16, the forward's output O is rounded to bf16
(relative 2^-9) before it enters D_i = dO_i . O_i, and its lse sums
bf16-rounded probabilities (relative error up to 2^-8); P_ij = exp(s_ij - lse_i)
and dS_ij then carry relative errors of a few 2^-9 against the exact values,
which the oracle uses, and a gradient entry sums many such terms of both signs,
so its error scales with the tensor's largest entries rather than its own.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import sparse_long_sequence_amd as la
from sparse_long_sequence_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL_ABS = {"f32": 2e-6, "bf16": 5e-3}  # times max |oracle| of the tensor
TOL_REL = {"f32": 2e-5, "bf16": 1e-2}  # times |oracle| of the entry
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    la.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rand(gen, shape, dtype):
    return torch.randn(shape, generator=gen).to(TORCH[dtype])


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check(tag, dtype, got, ref, names=("dq", "dk", "dv", "dqg", "dkg", "dvg"), floor=1e-30):
    """floor: the least scale a tensor is held to (for tensors that are zero in
    exact arithmetic, whose computed values are rounding noise)."""
    assert len(got) == len(ref)
    for name, g, r in zip(names, got, ref):
        g = g if isinstance(g, np.ndarray) else to64(g)
        scale = max(np.abs(r).max(), floor)
        err = np.abs(g - r)
        bound = TOL_ABS[dtype] * scale + TOL_REL[dtype] * np.abs(r)
        assert np.isfinite(g).all(), f"{tag} {name}: non-finite"
        say(f"{tag} {name}: max|err|/max|ref| = {err.max() / scale:.2e}, "
            f"worst err/bound = {(err / bound).max():.3f}")
        assert (err <= bound).all(), f"{tag} {name}: max err/bound {(err / bound).max()}"


def run_case(dev, tag, dtype, B, H, N, glob, R, dil, causal, sep, seg_rows, seed,
             inputs=None, floor=1e-30):
    say(f"backward {tag}: {dtype} B={B} H={H} N={N} |G|={len(glob)} R={R} dil={dil} "
        f"causal={causal} sep={sep} seg={seg_rows}")
    gen = torch.Generator().manual_seed(seed)
    if inputs is None:
        q, k, v = (rand(gen, (B, H, N, 64), dtype) for _ in range(3))
        qg, kg, vg = (rand(gen, (B, H, N, 64), dtype) for _ in range(3)) if sep else (None,) * 3
    else:
        q, k, v, qg, kg, vg = inputs
    dout = rand(gen, (B, H, N, 64), dtype)
    seg = None
    if seg_rows:
        # documents of the given lengths, one id each: the same for every batch
        # row, or (a tuple of tuples) one layout per batch row
        per_row = seg_rows if isinstance(seg_rows[0], tuple) else (seg_rows,) * B
        seg = torch.tensor(np.stack([
            np.concatenate([np.full(n, x, np.int32) for x, n in enumerate(lens)])
            for lens in per_row]))
    d = lambda t: None if t is None else t.to(dev).contiguous()
    gidx = torch.tensor(sorted(glob), dtype=torch.int32, device=dev) if glob else None
    out, lse = la.la_attn_forward(d(q), d(k), d(v), gidx, R, dil, causal, qg=d(qg), kg=d(kg),
                                  vg=d(vg), seg_ids=d(seg))
    grads = la.la_attn_backward(d(q), d(k), d(v), out, lse, d(dout), gidx, R, dil, causal,
                                qg=d(qg), kg=d(kg), vg=d(vg), seg_ids=d(seg))
    torch.cuda.synchronize()
    f64 = lambda t: None if t is None else to64(t)
    ref = oracle.attn_backward(f64(q), f64(k), f64(v), f64(dout), tuple(glob), R, dil, causal,
                               f64(qg), f64(kg), f64(vg),
                               seg=None if seg is None else seg.numpy())
    check(tag, dtype, grads, ref, floor=floor)
    return grads


CASES = [
    # tag, dtype, B, H, N, globals, R, dilation, causal, separate, segments
    ("shared", "bf16", 2, 2, 300, (0, 5, 100), 16, [1, 2], False, False, None),
    ("separate-causal", "bf16", 1, 2, 257, (3, 64, 65, 200), 8, [1, 3], True, True, None),
    ("segments", "bf16", 1, 3, 256, (0, 100, 200), 12, None, False, False, (100, 100, 56)),
    ("f32-causal", "f32", 1, 2, 200, (), 20, [1, 1], True, False, None),
    ("f32-separate", "f32", 1, 1, 130, (7, 64), 5, [2], False, True, None),
    ("dense-window", "bf16", 1, 2, 96, (), 96, None, False, False, None),
    ("no-window", "bf16", 1, 1, 128, (10, 11), 0, None, False, False, None),
    # six key (row) ranges for the global tiles; causal with late globals leaves
    # the last dK/dV range without rows (it still sweeps the global rows)
    ("ranges-causal", "bf16", 1, 2, 1500, (900, 1000, 1400), 32, [1, 2], True, True, None),
    ("ranges-shared", "bf16", 2, 1, 1100, tuple(range(0, 1100, 7)), 24, None, False, False, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_small(dev, case):
    tag, dtype, B, H, N, glob, R, dil, causal, sep, seg = case
    run_case(dev, tag, dtype, B, H, N, glob, R, dil, causal, sep, seg,
             seed=300 + CASES.index(case))


SEG_CASES = [
    # per-instance segment masks (packed documents, every pair masked): tag, B,
    # H, N, globals, R, dilation, causal, separate, documents (per row or shared)
    ("seg-globals-in-documents-sep", 2, 2, 700, (0, 1, 300, 301, 650), 40, (1, 2), False, True,
     ((300, 350, 50), (650, 50))),
    ("seg-causal-dilated", 1, 3, 513, (0, 200, 512), 33, (1, 2, 3), True, False,
     (1, 199, 250, 63)),
    # a tile-aligned layout (every tile of one document) and one of single
    # tokens: each row's only key is itself, so dS = 0 and dq = dk = 0 exactly
    # (held to the bar at unit scale, the inputs' and dv's magnitude)
    ("seg-aligned", 1, 2, 512, (0, 128, 256), 64, None, False, True, (128, 128, 256)),
    ("seg-singletons", 1, 1, 200, (5,), 8, None, False, False, tuple([1] * 200)),
    # the global tiles split over key (row) ranges
    ("seg-ranges", 1, 2, 1500, (0, 700, 701, 1499), 32, None, False, True, (700, 800)),
    ("seg-ranges-causal", 2, 2, 1300, tuple(range(0, 1300, 9)), 24, (1, 2), True, False,
     ((640, 660), (100, 1100, 100))),
]


@pytest.mark.parametrize("case", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_backward_segments(dev, case):
    """Pairs whose row and key lie in different segments are masked (ETC page,
    §3.4 "Per-instance attention masks"), for band, global-row and global-key
    pairs alike."""
    tag, B, H, N, G, R, dil, causal, sep, docs = case
    run_case(dev, tag, "bf16", B, H, N, G, R, None if dil is None else list(dil), causal, sep,
             docs, seed=600 + SEG_CASES.index(case),
             floor=1.0 if tag == "seg-singletons" else 1e-30)


def test_backward_segments_bias(dev):
    """Segment masks together with the scalar bias table."""
    w = W.Workload("seg-bias", B=2, H=2, N=900, radius=30, global_idx=(0, 1, 2, 450, 451),
                   dilation=(1, 2), separate_global=True, rel_k=5, rel_kind="scalar", seed=611)
    inp = W.make_inputs(w)
    inp.seg = torch.tensor(np.stack([np.repeat(np.arange(3), (450, 300, 150)),
                                     np.repeat(np.arange(2), (200, 700))]).astype(np.int32))
    run_label_case(dev, "seg-bias", "bf16", w, inp, seed=613)


def test_backward_packed(dev):
    """The packed-documents shape (B=2, H=12, N=4096 holding four documents of
    1024 tokens, R=256, the first 16 tokens of each document global with
    separate projections), every element against the oracle."""
    w = W.PACKED
    inp = W.make_inputs(w)
    run_case(dev, "packed", "bf16", w.B, w.H, w.N, w.global_idx, w.radius, None, w.causal, True,
             tuple(w.documents), seed=w.seed,
             inputs=(inp.q, inp.k, inp.v, inp.qg, inp.kg, inp.vg))


def test_backward_deterministic(dev):
    """Two calls give bitwise equal gradients (no atomics, fixed order)."""
    a = run_case(dev, "det-1", "bf16", 1, 2, 200, (0, 50), 10, None, False, True, None, seed=7)
    b = run_case(dev, "det-2", "bf16", 1, 2, 200, (0, 50), 10, None, False, True, None, seed=7)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # global tiles split over key (row) ranges whose partial sums are added
    a = run_case(dev, "det-3", "bf16", 1, 2, 1300, (0, 50, 1299), 10, None, False, True, None,
                 seed=8)
    b = run_case(dev, "det-4", "bf16", 1, 2, 1300, (0, 50, 1299), 10, None, False, True, None,
                 seed=8)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_longformer_base(dev):
    """The Longformer-base shape (B=2, H=12, N=4096, R=256, 64 global tokens with
    separate projections), every element against the oracle."""
    w = W.LONGFORMER_BASE
    inp = W.make_inputs(w)
    run_case(dev, "longformer-base", "bf16", w.B, w.H, w.N, w.global_idx, w.radius, None,
             w.causal, True, None, seed=w.seed,
             inputs=(inp.q, inp.k, inp.v, inp.qg, inp.kg, inp.vg))


def run_label_case(dev, tag, dtype, w: W.Workload, inp: W.Inputs, seed):
    """Forward then backward with the inputs' bias tables, label matrices and
    segment pieces; every gradient entry against the oracle's backward."""
    say(f"backward {tag}: {dtype} B={w.B} H={w.H} N={w.N} |G|={len(w.global_idx)} "
        f"R={w.radius} V={None if inp.rel_vec is None else inp.rel_vec.shape[1]} "
        f"pieces={inp.seg_pieces}")
    gen = torch.Generator().manual_seed(seed)
    dout = rand(gen, (w.B, w.H, w.N, 64), dtype)
    d = lambda t: None if t is None else t.to(dev).contiguous()
    gidx = torch.tensor(sorted(w.global_idx), dtype=torch.int32, device=dev)
    kw = dict(seg_ids=d(inp.seg), rel_vec=d(inp.rel_vec), rel_k=inp.rel_k,
              glabel=d(inp.glabel), llabel=d(inp.llabel), seg_pieces=inp.seg_pieces)
    sepkw = dict(qg=d(inp.qg), kg=d(inp.kg), vg=d(inp.vg))
    out, lse = la.la_attn_forward(d(inp.q), d(inp.k), d(inp.v), gidx, w.radius, w.dilation,
                                  w.causal, d(inp.rel_bias), **sepkw, **kw)
    grads = la.la_attn_backward(d(inp.q), d(inp.k), d(inp.v), out, lse, d(dout), gidx, w.radius,
                                w.dilation, w.causal, rel_bias=d(inp.rel_bias), **sepkw, **kw)
    torch.cuda.synchronize()
    f64 = lambda t: None if t is None else to64(t)
    np_ = lambda t: None if t is None else t.numpy()
    ref = oracle.attn_backward(f64(inp.q), f64(inp.k), f64(inp.v), f64(dout), w.global_idx,
                               w.radius, w.dilation, w.causal, f64(inp.qg), f64(inp.kg),
                               f64(inp.vg), seg=np_(inp.seg), rel_bias=f64(inp.rel_bias),
                               rel_vec=f64(inp.rel_vec), rel_k=inp.rel_k,
                               glabel=np_(inp.glabel), llabel=np_(inp.llabel),
                               seg_pieces=inp.seg_pieces)
    check(tag, dtype, grads, ref)


LABEL_CASES = [
    # tag, dtype, B, H, N, globals, R, dilation, causal, separate, rel_k, structural, kind, pieces
    ("bias-scalar", "bf16", 1, 2, 300, (0, 1, 150), 20, None, False, False, 5, 0, "scalar", 0),
    ("bias-both-sep", "bf16", 2, 2, 260, (3, 64, 200), 16, [1, 2], False, True, 3, 3, "both", 9),
    ("labels-f32-causal", "f32", 1, 2, 200, (5, 70, 71), 12, None, True, False, 2, 2, "vector", 6),
    ("labels-masks-only", "bf16", 1, 2, 230, (0, 100), 10, None, False, False, 0, 0, None, 4),
    # label matrices on the bf16 MFMA path: causal with separate projections and
    # the g2l and l2g pieces masked; dilated heads with vectors and every piece
    ("labels-bf16-causal-sep", "bf16", 1, 2, 300, (5, 70, 71, 200), 12, None, True, True, 3, 2,
     "both", 6),
    ("labels-vector-dilated", "bf16", 2, 3, 500, (0, 10, 250), 20, [1, 2, 3], False, False, 4, 3,
     "vector", 15),
]


@pytest.mark.parametrize("case", LABEL_CASES, ids=[c[0] for c in LABEL_CASES])
def test_backward_labels(dev, case):
    tag, dtype, B, H, N, G, R, dil, causal, sep, rk, ns, kind, pieces = case
    w = W.Workload(tag, B=B, H=H, N=N, dtype=dtype, radius=R, global_idx=G,
                   dilation=None if dil is None else tuple(dil), causal=causal,
                   separate_global=sep, seed=400 + LABEL_CASES.index(case))
    inp = W.make_inputs(w)
    V = 2 * rk + 1 + ns
    gen = torch.Generator().manual_seed(401)
    if kind in ("scalar", "both"):
        inp.rel_bias = 0.3 * torch.randn(H, V, generator=gen)
    if kind in ("vector", "both"):
        inp.rel_vec = 0.3 * torch.randn(H, V, 64, generator=gen)
    inp.rel_k = rk if kind else None
    rng = np.random.default_rng(403)
    vals = [0, V - 1, W.LABEL_DISTANCE, W.LABEL_DISTANCE, W.LABEL_MASKED] if kind else \
        [0, W.LABEL_DISTANCE, W.LABEL_MASKED]
    inp.glabel = torch.from_numpy(rng.choice(vals, size=(B, len(G), N)).astype(np.uint8))
    inp.llabel = torch.from_numpy(rng.choice(vals, size=(B, N, len(G))).astype(np.uint8))
    if pieces:
        inp.seg = torch.tensor((np.arange(N) * 3 // N)[None].repeat(B, 0), dtype=torch.int32)
        inp.seg_pieces = pieces
    run_label_case(dev, tag, dtype, w, inp, seed=405)


BIAS_CASES = [
    # the forward's scalar bias table alone (MFMA path): tag, B, H, N, globals,
    # R, dilation, causal, separate, rel_k
    ("bias-etc-like", 1, 3, 640, tuple(range(48)), 24, None, False, False, 6),
    ("bias-scattered-sep-causal", 1, 2, 700, (3, 64, 65, 300, 699), 20, (1, 2), True, True, 4),
    ("bias-no-window", 1, 1, 256, (10, 11), 0, None, False, False, 3),
    ("bias-windows-hold-globals", 2, 2, 1300, (100, 101, 640, 641, 642, 1299), 40, (1, 3), False,
     False, 12),
]


@pytest.mark.parametrize("case", BIAS_CASES, ids=[c[0] for c in BIAS_CASES])
def test_backward_bias_table(dev, case):
    """Same-kind pairs take the table's entry for their clipped distance (ETC
    page, §3.4 "Relative Position Encoding"); global tokens inside windows,
    dilated heads, separate projections and causal rows."""
    tag, B, H, N, G, R, dil, causal, sep, rk = case
    w = W.Workload(tag, B=B, H=H, N=N, radius=R, global_idx=G, dilation=dil, causal=causal,
                   separate_global=sep, rel_k=rk, rel_kind="scalar",
                   seed=500 + BIAS_CASES.index(case))
    inp = W.make_inputs(w)
    assert inp.rel_bias is not None and inp.rel_vec is None
    run_label_case(dev, tag, "bf16", w, inp, seed=501)


VEC_CASES = [
    # key-side label vectors on the MFMA path (the 2k+1 distance labels, no
    # label matrices): tag, B, H, N, globals, R, dilation, causal, separate,
    # rel_k, kind ("vector", or "both" with the scalar table), documents
    ("vec-etc-like", 1, 3, 640, tuple(range(48)), 24, None, False, False, 6, "vector", None),
    # (the first global token at 40, not 3: under causal masking a global row
    # at 3 sees four keys whose dS terms are of order one and sum to zero, so
    # the bf16 rounding of dS for the MFMAs, and of O in D_i, leaves an error
    # set by sum_j |dS_ij| |k_j| rather than by the tensor's largest entry; an
    # fp64 emulation of exactly those two roundings puts that row at 1.3-1.6x
    # the bar, as the kernel measured)
    ("vec-both-scattered-sep-causal", 1, 2, 700, (40, 64, 65, 300, 699), 20, (1, 2), True, True,
     4, "both", None),
    ("vec-no-window", 1, 1, 256, (10, 11), 0, None, False, False, 3, "vector", None),
    ("vec-windows-hold-globals", 2, 2, 1300, (100, 101, 640, 641, 642, 1299), 40, (1, 3), False,
     False, 12, "vector", None),
    # labels wider than the window: interior labels no pair reaches
    ("vec-k-above-radius", 1, 2, 300, (0, 150), 5, None, False, True, 9, "both", None),
    ("vec-segments", 2, 2, 900, (0, 1, 2, 450, 451), 30, (1, 2), False, True, 5, "vector",
     (450, 300, 150)),
    # no global token at all (no tile carries global flags), causal, ragged tail
    ("vec-no-globals-causal", 1, 2, 500, (), 30, None, True, False, 7, "vector", None),
]


@pytest.mark.parametrize("case", VEC_CASES, ids=[c[0] for c in VEC_CASES])
def test_backward_label_vectors(dev, case):
    """Same-kind pairs' logits take q_i . a_l / sqrt(D) for their clipped
    distance label (ETC page, §3.4 "Relative Position Encoding"), and dq_i the
    term sum_j dS_ij a_l; with the scalar table too ("both"), segments, global
    tokens inside windows, dilated heads, separate projections and causal rows."""
    tag, B, H, N, G, R, dil, causal, sep, rk, kind, docs = case
    w = W.Workload(tag, B=B, H=H, N=N, radius=R, global_idx=G, dilation=dil, causal=causal,
                   separate_global=sep, rel_k=rk, rel_kind=kind,
                   seed=700 + VEC_CASES.index(case))
    inp = W.make_inputs(w)
    assert inp.rel_vec is not None and inp.glabel is None and inp.llabel is None
    if docs:
        inp.seg = torch.tensor(np.repeat(np.arange(len(docs)), docs)[None].repeat(B, 0)
                               .astype(np.int32))
    run_label_case(dev, tag, "bf16", w, inp, seed=701)


def test_backward_label_vectors_deterministic(dev):
    """Two calls with label vectors give bitwise equal gradients (the label
    sums add in a fixed order)."""
    w = W.Workload("vec-det", B=1, H=2, N=700, radius=30, global_idx=(0, 1, 350),
                   separate_global=True, rel_k=8, rel_kind="both", seed=720)
    inp = W.make_inputs(w)
    d = lambda t: None if t is None else t.to(dev).contiguous()
    gidx = torch.tensor(w.global_idx, dtype=torch.int32, device=dev)
    kw = dict(qg=d(inp.qg), kg=d(inp.kg), vg=d(inp.vg), rel_vec=d(inp.rel_vec), rel_k=inp.rel_k)
    out, lse = la.la_attn_forward(d(inp.q), d(inp.k), d(inp.v), gidx, w.radius, None, False,
                                  d(inp.rel_bias), **kw)
    dout = rand(torch.Generator().manual_seed(721), (1, 2, 700, 64), "bf16").to(dev)
    g1 = la.la_attn_backward(d(inp.q), d(inp.k), d(inp.v), out, lse, dout, gidx, w.radius,
                             rel_bias=d(inp.rel_bias), **kw)
    g2 = la.la_attn_backward(d(inp.q), d(inp.k), d(inp.v), out, lse, dout, gidx, w.radius,
                             rel_bias=d(inp.rel_bias), **kw)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_backward_etc_vectors(dev):
    """The ETC global-local shape with key-side label vectors (B=1, H=12,
    n_g=256 then n_l=4096, R=84, per-head vectors for distances in [-12, 12]),
    every element against the oracle."""
    w = W.WORKLOADS["etc-ng256-nl4096-r84-relvec12"]
    run_label_case(dev, "etc-vectors", "bf16", w, W.make_inputs(w), seed=w.seed)


def test_backward_etc_shape(dev):
    """The ETC global-local shape (B=1, H=12, n_g=256 global tokens then
    n_l=4096 long tokens, R=84, per-head scalar table for distances in
    [-12, 12]), every element against the oracle."""
    w = W.WORKLOADS["etc-ng256-nl4096-r84-relk12"]
    run_label_case(dev, "etc-shape", "bf16", w, W.make_inputs(w), seed=w.seed)


def test_backward_etc_structured(dev):
    """The ETC structured layout (hard g2l, no cross-context g2g or l2l, four
    structural labels, key-side label vectors) at a reduced size."""
    w = W.Workload("etc-structured-bwd", B=1, H=2, N=64 + 900, radius=40,
                   global_idx=tuple(range(64)), rel_k=6, rel_kind="both", structure=(4, 3),
                   seed=407)
    run_label_case(dev, "etc-structured", "bf16", w, W.make_inputs(w), seed=409)


def test_backward_etc_structured_full(dev):
    """The full ETC structured workload (B=1, H=12, 256 global tokens then 4096
    long tokens, R=84, 16 contexts and 7 answer candidates: label matrices, hard
    g2l and g2g masks, l2l segment ids, 29 labels with key-side vectors), every
    element against the oracle."""
    w = W.WORKLOADS["etc-structured-ng256-nl4096-r84-relvec12-v29"]
    run_label_case(dev, "etc-structured-full", "bf16", w, W.make_inputs(w), seed=w.seed)


def test_backward_graph_replay(dev):
    """The backward call captured in a HIP graph (it writes its whole workspace
    with kernels, no memset) and replayed, with eager work between replays:
    every replay equals the eager result bit for bit."""
    gen = torch.Generator().manual_seed(31)
    B, H, N = 1, 2, 320
    q, k, v, dout = (rand(gen, (B, H, N, 64), "bf16").to(dev) for _ in range(4))
    g = torch.tensor([0, 7, 200], dtype=torch.int32, device=dev)
    out, lse = la.la_attn_forward(q, k, v, g, 24, [1, 2], True)
    call = la.bind_attn_backward(q, k, v, out, lse, dout, g, 24, [1, 2], True)
    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in call.grads]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call_s = la.bind_attn_backward(q, k, v, out, lse, dout, g, 24, [1, 2], True, stream=s)
        call_s()  # warm-up on the capture stream
        s.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            call_s()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in call_s.grads:
            t.fill_(float("nan"))
        la.la_attn_forward(k, q, v, g, 8)  # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip(call_s.grads, eager):
            assert torch.equal(x, y), f"replay {rep} differs"


def test_backward_empty_batch(dev):
    q = torch.empty(0, 2, 64, 64, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(0, 2, 64, dtype=torch.float32, device=dev)
    grads = la.la_attn_backward(q, q, q, q, lse, q, None, 4)
    assert len(grads) == 3 and all(t.numel() == 0 for t in grads)


LONGNET_CASES = [
    # tag, B, H, N, pairs, causal
    ("causal", 1, 4, 512, ((128, 1), (256, 2), (512, 4)), True),
    ("non-causal", 2, 3, 384, ((64, 1), (192, 3)), False),
    ("ragged-last-segment", 1, 6, 600, ((256, 1), (512, 2), (600, 6)), True),
    ("n4096", 1, 2, 4096, ((1024, 1), (2048, 2), (4096, 4)), True),
    # no dilation-1 pattern: rows that no pattern covers have lse = -inf and no gradient
    ("no-r1-uncovered", 1, 5, 333, ((64, 2), (128, 3), (333, 5)), True),
    # the dilation-1 pattern (launched first, storing) is not the first given
    ("r1-not-first", 1, 3, 700, ((256, 2), (128, 1), (700, 7)), False),
]


@pytest.mark.parametrize("case", LONGNET_CASES, ids=[c[0] for c in LONGNET_CASES])
def test_backward_longnet(dev, case):
    """The LongNet mixture's backward against the oracle's multiplicity-weighted
    chain rule; the forward supplies out and its mixture lse."""
    tag, B, H, N, pairs, causal = case
    say(f"longnet backward {tag}: B={B} H={H} N={N} pairs={pairs} causal={causal}")
    gen = torch.Generator().manual_seed(400 + LONGNET_CASES.index(case))
    q, k, v, dout = (rand(gen, (B, H, N, 64), "bf16") for _ in range(4))
    d = lambda t: t.to(dev).contiguous()
    w, r = [p[0] for p in pairs], [p[1] for p in pairs]
    out, lse = la.la_dilated_forward(d(q), d(k), d(v), w, r, causal)
    grads = la.la_dilated_backward(d(q), d(k), d(v), out, lse, d(dout), w, r, causal)
    torch.cuda.synchronize()
    ref = oracle.longnet_backward(to64(q), to64(k), to64(v), to64(dout), pairs, causal)
    check(f"longnet-{tag}", "bf16", grads, ref)
    if all(r_ > 1 for r_ in r):
        # a row no pattern keeps: for head h, offset h mod r differs from the
        # row's residue in every pattern's segment
        mult = [oracle.longnet_mult_rows(N, h, pairs, causal) for h in range(H)]
        unc = np.array([[m[i].sum() == 0 for i in range(N)] for m in mult])
        assert unc.any()
        assert np.isneginf(to64(lse)[:, unc]).all()
        assert (to64(grads[0])[:, unc] == 0).all(), "uncovered rows must get dq = 0"


def _segment_end_keys(w, h):
    """Keys j at the ends of the 8192-aligned segments that the (32768, 12)
    pattern does not keep for head h (and the sequence's last keys): causal
    rows attend them only from the same short tail of each segment, so the
    oracle evaluates few rows per key."""
    keys = []
    for end in range(8192, w.N + 1, 8192):
        for t in (0, 1, 2, 5, 17, 40):
            j = end - 1 - t
            if end == w.N or (j % 12) != (h % 12):
                keys.append(j)
    return keys


def test_backward_longnet_full_shape(dev):
    """The LongNet workload's own shape (B=1, H=12, N=32768, five patterns,
    causal), heads 0, 5 and 11 (distinct offsets under every pattern): dq of
    every tile-edge row of those heads' segments and some random rows, dk and dv
    of keys at segment ends, against the oracle's chosen-output gradients; and,
    over every key of those heads, the two sums the chain rule fixes: sum_j dk_j
    = 0 and sum_j dv_j = sum_i dO_i (every row is covered: a pattern has r = 1)."""
    w = W.LONGNET_SHARE
    inp = W.make_inputs(w)
    dout = torch.randn(inp.q.shape, generator=torch.Generator().manual_seed(410)).to(torch.bfloat16)
    d = lambda t: t.to(dev).contiguous()
    seg, dil = [p[0] for p in w.pairs], [p[1] for p in w.pairs]
    say(f"longnet backward full shape: B={w.B} H={w.H} N={w.N} pairs={w.pairs}")
    out, lse = la.la_dilated_forward(d(inp.q), d(inp.k), d(inp.v), seg, dil, True)
    grads = la.la_dilated_backward(d(inp.q), d(inp.k), d(inp.v), out, lse, d(dout), seg, dil, True)
    torch.cuda.synchronize()
    g64 = [to64(t) for t in grads]
    rng = np.random.default_rng(411)
    rows, keys = [], []
    for h in (0, 5, 11):
        edge = sorted({x for t in range(0, w.N, 2048) for x in (t, t + 1, t + 63, t + 64,
                                                                 t + 2047)})
        for i in edge + rng.integers(0, w.N, 24).tolist():
            rows.append((0, h, i))
        keys += [(0, h, j) for j in _segment_end_keys(w, h)]
    rows, keys = np.array(rows), np.array(keys)
    f = lambda t: t.to(torch.float64).numpy()
    dq_ref, dk_ref, dv_ref = oracle.longnet_backward_sel(f(inp.q), f(inp.k), f(inp.v), f(dout),
                                                         w.pairs, True, rows=rows, keys=keys)
    pick = lambda g, s: g[s[:, 0], s[:, 1], s[:, 2]]
    check("longnet-full-dq", "bf16", [pick(g64[0], rows)], [dq_ref], names=("dq",))
    check("longnet-full-dkv", "bf16", [pick(g64[1], keys), pick(g64[2], keys)], [dk_ref, dv_ref],
          names=("dk", "dv"))
    do64 = to64(dout)
    for h in (0, 5, 11):
        dk_sum = g64[1][0, h].sum(0)
        dk_mag = np.abs(g64[1][0, h]).sum(0)
        assert (np.abs(dk_sum) <= 1e-3 * dk_mag + 1e-6).all(), f"h={h}: sum of dk is not 0"
        dv_sum, do_sum = g64[2][0, h].sum(0), do64[0, h].sum(0)
        assert np.abs(dv_sum - do_sum).max() <= 2e-2 * np.abs(do64[0, h]).sum(0).max() / 64, \
            f"h={h}: sum of dv differs from sum of dO"
