"""Structured inputs on the GPU against the fp64 oracle: per-pair label
matrices and segment masks restricted to some pieces (ETC page, 3.4
"Per-instance attention masks", "How Global-Local Attention Encodes Structured
Inputs" and "Relative Position Encoding", Step 1 and its implementation note).

Every row is compared at sizes that span several query and key tiles with
ragged tails: an ETC layout (globals first, one run) built by the seeded
structure recipe, scattered global tokens with random labels (every kind of
label value, separate global projections, a dilated head, causal), labels
without any table (pure masks), each piece subset of the segment mask on
packed documents, fp32, and an exact-mask check (Q = 0, one-hot V) of the
label masks.
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

TOL = {"f32": 1e-4, "bf16": 2e-2}
LSE_TOL = {"f32": 1e-4, "bf16": 2.0 ** -8 + 1e-4}
DIST, MASK = W.LABEL_DISTANCE, W.LABEL_MASKED


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    la.lib()
    return torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def run_both(w, inp, dev):
    """The GPU call and the oracle on the same inputs (every row)."""
    g = torch.tensor(w.global_idx, dtype=torch.int32, device=dev) if w.global_idx else None
    d = lambda t: None if t is None else t.to(dev)
    out, lse = la.la_attn_forward(d(inp.q), d(inp.k), d(inp.v), g, w.radius, w.dilation,
                                  w.causal, d(inp.rel_bias), qg=d(inp.qg), kg=d(inp.kg),
                                  vg=d(inp.vg), rel_vec=d(inp.rel_vec), seg_ids=d(inp.seg),
                                  rel_k=inp.rel_k, glabel=d(inp.glabel), llabel=d(inp.llabel),
                                  seg_pieces=inp.seg_pieces)
    torch.cuda.synchronize()
    np_ = lambda t: None if t is None else t.numpy()
    o_ref, l_ref = oracle.attn_rows(to64(inp.q), to64(inp.k), to64(inp.v), w.global_idx,
                                    w.radius, w.dilation, w.causal, to64(inp.rel_bias),
                                    to64(inp.qg), to64(inp.kg), to64(inp.vg),
                                    rel_vec=to64(inp.rel_vec), seg=np_(inp.seg), rel_k=inp.rel_k,
                                    glabel=np_(inp.glabel), llabel=np_(inp.llabel),
                                    seg_pieces=inp.seg_pieces)
    return out, lse, o_ref, l_ref


def compare(tag, dtype, out, lse, o_ref, l_ref):
    o, l = to64(out), to64(lse)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin), f"{tag}: lse finiteness differs"
    err = np.abs(o - o_ref).max()
    lerr = np.abs(l[fin] - l_ref[fin]).max() if fin.any() else 0.0
    say(f"{tag}: max|dO| = {err:.3e}  max|dlse| = {lerr:.3e}  rows without keys: {(~fin).sum()}")
    assert err <= TOL[dtype], f"{tag}: max|dO| {err}"
    assert lerr <= LSE_TOL[dtype], f"{tag}: max|dlse| {lerr}"


# --------------------------------------------------------------------------
# the ETC structured layout (seeded recipe), several sizes, dtypes and tables
# --------------------------------------------------------------------------
ETC_CASES = [
    # name, B, H, n_global, n_long, R, (contexts, candidates), rel_k, rel_kind, dtype
    ("etc-struct-vec", 2, 2, 64, 1500, 40, (4, 3), 4, "vector", "bf16"),
    ("etc-struct-both-ragged", 1, 3, 77, 1203, 84, (5, 2), 12, "both", "bf16"),
    ("etc-struct-scalar-f32", 1, 2, 40, 700, 30, (3, 2), 3, "scalar", "f32"),
    ("etc-struct-many-globals", 1, 2, 300, 1400, 25, (10, 9), 6, "vector", "bf16"),
]


@pytest.mark.parametrize("case", ETC_CASES, ids=[c[0] for c in ETC_CASES])
def test_etc_structured(dev, case):
    name, B, H, ng, nl, R, st, rk, kind, dt = case
    w = W.Workload(name, B=B, H=H, N=ng + nl, dtype=dt, radius=R, global_idx=tuple(range(ng)),
                   rel_k=rk, rel_kind=kind, structure=st, seed=131)
    inp = W.make_inputs(w)
    say(f"case {name}: B={B} H={H} N={w.N} n_global={ng} R={R} V={2 * rk + 5} {dt}")
    out, lse, o_ref, l_ref = run_both(w, inp, dev)
    compare(name, dt, out, lse, o_ref, l_ref)


# --------------------------------------------------------------------------
# scattered global tokens with random labels of every kind
# --------------------------------------------------------------------------
def _random_labels(rng, B, N, G, V, extra=()):
    vals = [0, 1, V - 1, V - 2, DIST, DIST, DIST, MASK, 200, *extra]
    glabel = rng.choice(vals, size=(B, len(G), N)).astype(np.uint8)
    llabel = rng.choice(vals, size=(B, N, len(G))).astype(np.uint8)
    return torch.from_numpy(glabel), torch.from_numpy(llabel)


SCATTER_CASES = [
    # name, B, H, N, R, G, dilation, causal, separate, rel_k, n_struct, rel_kind, dtype
    ("scatter-sep-dil", 2, 2, 700, 33, (0, 63, 64, 65, 127, 300, 301, 511, 699), (1, 2), False,
     True, 3, 3, "both", "bf16"),
    ("scatter-causal", 1, 3, 515, 50, (1, 2, 3, 200, 514), None, True, False, 5, 2, "vector",
     "bf16"),
    ("scatter-f32", 2, 2, 333, 20, (5, 70, 71, 140, 332), (1, 3), False, True, 2, 4, "scalar",
     "f32"),
    # globals first (one run): labels through the contiguous global tiles
    ("run-both", 1, 2, 600, 40, tuple(range(100)), None, False, False, 4, 3, "both", "bf16"),
]


@pytest.mark.parametrize("case", SCATTER_CASES, ids=[c[0] for c in SCATTER_CASES])
def test_labels_scattered(dev, case):
    name, B, H, N, R, G, dil, causal, sep, rk, ns, kind, dt = case
    w = W.Workload(name, B=B, H=H, N=N, dtype=dt, radius=R, global_idx=G, dilation=dil,
                   causal=causal, separate_global=sep, seed=137)
    inp = W.make_inputs(w)
    V = 2 * rk + 1 + ns
    gen = torch.Generator().manual_seed(139)
    if kind in ("scalar", "both"):
        inp.rel_bias = 0.3 * torch.randn(H, V, generator=gen)
    if kind in ("vector", "both"):
        inp.rel_vec = 0.3 * torch.randn(H, V, w.D, generator=gen)
    inp.rel_k = rk
    inp.glabel, inp.llabel = _random_labels(np.random.default_rng(141), B, N, G, V)
    say(f"case {name}: B={B} H={H} N={N} |G|={len(G)} V={V} causal={causal} {dt}")
    out, lse, o_ref, l_ref = run_both(w, inp, dev)
    compare(name, dt, out, lse, o_ref, l_ref)


def test_labels_without_tables(dev):
    # label matrices as pure masks: 0 keeps a pair (no table, no bias), the
    # distance label keeps it, anything else masks it; only one of the two
    # matrices given
    G = (0, 1, 2, 100, 250)
    w = W.Workload("labels-masks-only", B=2, H=2, N=400, radius=30, global_idx=G, seed=143)
    rng = np.random.default_rng(145)
    for which in ("glabel", "llabel", "both"):
        inp = W.make_inputs(w)
        gl, ll = _random_labels(rng, w.B, w.N, G, 1)
        inp.glabel = gl if which in ("glabel", "both") else None
        inp.llabel = ll if which in ("llabel", "both") else None
        say(f"case labels-masks-only/{which}")
        out, lse, o_ref, l_ref = run_both(w, inp, dev)
        compare(f"labels-masks-only/{which}", w.dtype, out, lse, o_ref, l_ref)


def test_wide_table_without_matrices(dev):
    # a vocabulary wider than the 2k+1 distance labels but no label matrix:
    # only the distance labels are reached, from tables of V entries per head
    G = (0, 1, 2, 100, 250)
    w = W.Workload("wide-table", B=1, H=3, N=400, radius=30, global_idx=G, seed=159)
    inp = W.make_inputs(w)
    gen = torch.Generator().manual_seed(161)
    inp.rel_k, V = 4, 13
    inp.rel_bias = 0.3 * torch.randn(3, V, generator=gen)
    inp.rel_vec = 0.3 * torch.randn(3, V, w.D, generator=gen)
    say("case wide-table")
    out, lse, o_ref, l_ref = run_both(w, inp, dev)
    compare("wide-table", w.dtype, out, lse, o_ref, l_ref)


# --------------------------------------------------------------------------
# segment masks on some pieces only
# --------------------------------------------------------------------------
PIECES = [1, 2, 4, 8, 3, 12, 5, 10, 6, 9, 14, 15]


@pytest.mark.parametrize("pieces", PIECES, ids=[f"pieces{p}" for p in PIECES])
def test_segment_pieces(dev, pieces):
    # packed documents of different lengths, globals in several documents and
    # at tile edges; a dilated head
    G = (0, 1, 64, 300, 301, 640, 899)
    w = W.Workload(f"pieces-{pieces}", B=2, H=2, N=900, radius=60, dilation=(1, 2),
                   global_idx=G, rel_k=3, rel_kind="scalar", seed=147)
    inp = W.make_inputs(w)
    inp.seg = torch.tensor(np.stack([np.repeat([0, 1, 2], [300, 340, 260]),
                                     np.repeat([5, 6], [640, 260])]), dtype=torch.int32)
    inp.seg_pieces = pieces
    say(f"case pieces={pieces}")
    out, lse, o_ref, l_ref = run_both(w, inp, dev)
    compare(f"pieces-{pieces}", w.dtype, out, lse, o_ref, l_ref)


def test_segment_pieces_f32_causal_labels(dev):
    # pieces with labels, fp32, causal, scattered globals
    G = (3, 90, 91, 300)
    w = W.Workload("pieces-f32-causal", B=1, H=2, N=420, dtype="f32", radius=35, causal=True,
                   global_idx=G, seed=149)
    inp = W.make_inputs(w)
    inp.seg = torch.tensor((np.arange(420) // 97)[None], dtype=torch.int32)
    inp.seg_pieces = 9  # g2g and l2l
    inp.rel_k, V = 2, 8
    inp.rel_vec = 0.3 * torch.randn(2, V, w.D, generator=torch.Generator().manual_seed(151))
    inp.glabel, inp.llabel = _random_labels(np.random.default_rng(153), 1, 420, G, V)
    say("case pieces-f32-causal")
    out, lse, o_ref, l_ref = run_both(w, inp, dev)
    compare("pieces-f32-causal", w.dtype, out, lse, o_ref, l_ref)


# --------------------------------------------------------------------------
# exact label masks: Q = 0 and V = one-hot(j mod D) make each output row the
# uniform average over the row's allowed keys, so a pair wrongly kept or
# dropped shows as an error of at least 1 / (keys + 1)
# --------------------------------------------------------------------------
def test_label_masks_exact(dev):
    G = tuple(range(48)) + (500, 777)
    w = W.Workload("label-masks-exact", B=2, H=2, N=1000, radius=70, global_idx=G,
                   structure=(), seed=155)
    B, H, N, D = w.B, w.H, w.N, w.D
    inp = W.make_inputs(w)
    inp.q = torch.zeros(B, H, N, D, dtype=torch.bfloat16)
    v = torch.zeros(B, H, N, D)
    v[:, :, torch.arange(N), torch.arange(N) % D] = 1
    inp.v = v.to(torch.bfloat16)
    rng = np.random.default_rng(157)
    gl = rng.choice([DIST, MASK], p=[0.7, 0.3], size=(B, len(G), N)).astype(np.uint8)
    ll = rng.choice([DIST, MASK, 0], p=[0.5, 0.3, 0.2], size=(B, N, len(G))).astype(np.uint8)
    gl[0, 5, :] = MASK        # a global row with no allowed key: zeros, lse = -inf
    gl[1, 7, :] = MASK
    gl[1, 7, 900] = DIST      # ... and one with a single key
    inp.glabel, inp.llabel = torch.from_numpy(gl), torch.from_numpy(ll)
    inp.seg = torch.tensor(np.stack([np.repeat([0, 1], [600, 400])] * B), dtype=torch.int32)
    inp.seg_pieces = 8
    say("case label-masks-exact")
    out, lse, o_ref, l_ref = run_both(w, inp, dev)
    o, l = to64(out), to64(lse)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin)
    assert not fin[0, :, 5].any() and np.all(o[0, :, 5] == 0)
    # lse = log(count) exactly up to the bf16 rounding of nothing (all logits 0)
    cnt_ref = np.rint(np.exp(l_ref[fin]))
    cnt = np.rint(np.exp(l[fin]))
    assert np.array_equal(cnt, cnt_ref), "allowed key counts differ"
    err = np.abs(o - o_ref).max()
    say(f"label-masks-exact: max|dO| = {err:.3e}")
    assert err < 1.0 / (2 * (cnt_ref.max() + 1))
