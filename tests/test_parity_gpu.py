"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Tolerances: max |O_gpu - O_oracle| <= 1e-4 for fp32 inputs and <= 2e-2 for bf16
inputs (fp32 accumulation). lse within 1e-4 for fp32 inputs. For bf16 inputs the
kernel rounds each probability p to bf16 (the operand of the PV product) and
normalises by the sum of the rounded values, so the row sum carries a relative
error of at most 2^-8 (bf16 unit roundoff: 8 significant bits, round to nearest)
and lse an absolute error of at most ln(1 + 2^-8) < 2^-8: lse within 2^-8 + 1e-4
for bf16 (the second term is the fp32 allowance).
Mask and global-index handling are checked exactly: with Q = 0 every logit is
0, so exp(lse_i) is the number of allowed keys of row i (the multiplicity sum
for LongNet); with V = one-hot(j mod 64), O_i[c] * count_i is the number of
allowed keys congruent to c mod 64.
"""
from __future__ import annotations

import math
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


def label_kw(inp: W.Inputs, dev=None):
    """Structural labels and piece-selected segment masks of the inputs, if any."""
    if inp.glabel is None and inp.llabel is None and not inp.seg_pieces:
        return {}
    cv = (lambda t: None if t is None else t.to(dev)) if dev is not None else \
        (lambda t: None if t is None else t.numpy())
    return dict(glabel=cv(inp.glabel), llabel=cv(inp.llabel), seg_pieces=inp.seg_pieces,
                rel_k=inp.rel_k)


def gpu_attn(w: W.Workload, inp: W.Inputs, dev, **kw):
    g = torch.tensor(w.global_idx, dtype=torch.int32, device=dev) if w.global_idx else None
    d = lambda t: None if t is None else t.to(dev)
    kw = {**label_kw(inp, dev), **kw}
    out, lse = la.la_attn_forward(d(inp.q), d(inp.k), d(inp.v), g, w.radius, w.dilation, w.causal,
                                  d(inp.rel_bias), qg=d(inp.qg), kg=d(inp.kg), vg=d(inp.vg),
                                  rel_vec=d(inp.rel_vec), seg_ids=d(inp.seg), **kw)
    torch.cuda.synchronize()
    return out, lse


def gpu_dilated(w: W.Workload, inp: W.Inputs, dev):
    out, lse = la.la_dilated_forward(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev),
                                     [p[0] for p in w.pairs], [p[1] for p in w.pairs], w.causal)
    torch.cuda.synchronize()
    return out, lse


def oracle_attn(w: W.Workload, inp: W.Inputs, sel=None):
    return oracle.attn_rows(to64(inp.q), to64(inp.k), to64(inp.v), w.global_idx, w.radius,
                            w.dilation, w.causal, to64(inp.rel_bias), to64(inp.qg), to64(inp.kg),
                            to64(inp.vg), sel=sel, rel_vec=to64(inp.rel_vec),
                            seg=None if inp.seg is None else inp.seg.numpy(), **label_kw(inp))


def gpu_fixed(w: W.Workload, inp: W.Inputs, dev):
    out, lse = la.la_fixed_forward(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), w.fixed[0],
                                   w.fixed[1], w.causal)
    torch.cuda.synchronize()
    return out, lse


def oracle_fixed(w: W.Workload, inp: W.Inputs, sel=None):
    return oracle.fixed_rows(to64(inp.q), to64(inp.k), to64(inp.v), w.fixed[0], w.fixed[1],
                             w.causal, sel=sel)


def oracle_dilated(w: W.Workload, inp: W.Inputs, sel=None):
    return oracle.longnet_rows(to64(inp.q), to64(inp.k), to64(inp.v), w.pairs, w.causal, sel=sel)


def compare(w, out, lse, o_ref, l_ref, sel=None, tag=""):
    o = to64(out)
    l = to64(lse)
    if sel is not None:
        s = np.asarray(sel)
        o = o[s[:, 0], s[:, 1], s[:, 2]]
        l = l[s[:, 0], s[:, 1], s[:, 2]]
    err = np.abs(o - o_ref).max()
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin), f"{tag}: lse finiteness differs"
    lerr = np.abs(l[fin] - l_ref[fin]).max() if fin.any() else 0.0
    say(f"{tag}: max|dO| = {err:.3e}  max|dlse| = {lerr:.3e}")
    assert err <= TOL[w.dtype], f"{tag}: max|dO| {err} > {TOL[w.dtype]}"
    assert lerr <= LSE_TOL[w.dtype], f"{tag}: max|dlse| {lerr} > {LSE_TOL[w.dtype]}"


# --------------------------------------------------------------------------
# small cases: several tiles, ragged tails, every feature; all rows compared
# --------------------------------------------------------------------------
SMALL = [
    # name, N, H, R, dilation, causal, G, rel_k, separate, dtype
    ("band-ragged", 300, 2, 37, None, False, (), 0, False, "bf16"),
    ("band-f32", 300, 2, 37, None, False, (), 0, False, "f32"),
    ("band-R0", 130, 1, 0, None, False, (), 0, False, "bf16"),
    ("band-R>=N", 100, 2, 150, None, False, (), 0, False, "bf16"),
    ("band-N1", 1, 1, 3, None, False, (), 0, False, "bf16"),
    ("band-N<64", 45, 2, 7, None, True, (), 0, False, "f32"),
    ("global-scatter", 333, 3, 20, None, False, (0, 5, 64, 65, 200, 332), 0, False, "bf16"),
    ("global-sep-f32", 257, 2, 30, None, False, (1, 2, 3, 100, 256), 0, True, "f32"),
    ("global-sep-bf16", 257, 2, 30, None, False, tuple(range(70)), 0, True, "bf16"),
    ("causal-global", 200, 2, 25, None, True, (0, 63, 64, 150), 0, False, "bf16"),
    ("dilated-mix", 301, 4, 19, (1, 2, 3, 5), False, (), 0, False, "bf16"),
    ("dilated-causal-global", 301, 4, 19, (1, 2, 3, 5), True, (7, 90, 91), 0, False, "bf16"),
    ("dilated-global-f32", 150, 2, 9, (3, 1), False, (0, 149), 0, False, "f32"),
    ("relbias", 400, 3, 21, None, False, tuple(range(30)), 5, False, "bf16"),
    ("relbias-f32-causal", 260, 2, 40, (1, 2), True, (3, 77, 200), 12, False, "f32"),
    ("relbias-sep", 300, 2, 33, None, False, (0, 1, 2, 150, 299), 3, True, "bf16"),
    ("relbias-dil-causal", 350, 4, 17, (1, 2, 3, 4), True, (5, 64, 65, 200, 349), 7, False, "bf16"),
    ("all-global", 96, 1, 2, None, False, tuple(range(96)), 0, False, "bf16"),
    # ETC key-side label vectors (rel_k > 0 with a kind): alone, with the scalar table, fp32,
    # separate projections, causal and dilated windows
    ("relvec", 400, 3, 21, None, False, tuple(range(30)), (5, "vector"), False, "bf16"),
    ("relvec-both-sep", 300, 2, 33, None, False, (0, 1, 2, 150, 299), (3, "both"), True, "bf16"),
    ("relvec-f32-causal", 260, 2, 40, (1, 2), True, (3, 77, 200), (12, "vector"), False, "f32"),
    ("relvec-dil-causal", 350, 4, 17, (1, 2, 3, 4), True, (5, 64, 65, 200, 349), (7, "both"),
     False, "bf16"),
    ("relvec-etc-like", 544, 2, 10, None, False, tuple(range(32)), (12, "vector"), False, "bf16"),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_band_global(dev, case):
    name, N, H, R, dil, causal, G, rk, sep, dt = case
    kind = "scalar"
    if isinstance(rk, tuple):
        rk, kind = rk
    w = W.Workload(name, B=2, H=H, N=N, dtype=dt, radius=R, global_idx=G, dilation=dil,
                   causal=causal, rel_k=rk, rel_kind=kind, separate_global=sep, seed=77)
    inp = W.make_inputs(w)
    say(f"case {name}: N={N} H={H} R={R} dil={dil} causal={causal} |G|={len(G)} rel_k={rk} "
        f"sep={sep} {dt}")
    out, lse = gpu_attn(w, inp, dev)
    o_ref, l_ref = oracle_attn(w, inp)
    compare(w, out, lse, o_ref, l_ref, tag=name)


SMALL_DIL = [
    ("longnet-small", 256, 7, ((16, 1), (32, 2), (64, 4), (96, 6)), True),
    ("longnet-ragged", 300, 5, ((64, 1), (128, 3), (300, 12)), True),
    ("longnet-noncausal", 200, 3, ((50, 1), (100, 4)), False),
    ("longnet-uncovered", 128, 2, ((64, 2),), True),
    ("longnet-dense", 190, 2, ((190, 1),), True),
    ("longnet-multitile", 1000, 3, ((400, 1), (1000, 2)), True),
    # no dilation-1 pattern: every pattern writes partials, a combine launch mixes
    ("longnet-no-finisher", 333, 5, ((64, 2), (128, 3), (333, 5)), True),
    # the dilation-1 pattern listed after others, and a second one among the partials
    ("longnet-finisher-order", 400, 4, ((128, 2), (64, 1), (200, 1), (400, 4)), True),
]


@pytest.mark.parametrize("case", SMALL_DIL, ids=[c[0] for c in SMALL_DIL])
def test_small_dilated(dev, case):
    name, N, H, pairs, causal = case
    w = W.Workload(name, B=2, H=H, N=N, kind="dilated", causal=causal, pairs=pairs, seed=78)
    inp = W.make_inputs(w)
    say(f"case {name}: N={N} H={H} pairs={pairs} causal={causal}")
    out, lse = gpu_dilated(w, inp, dev)
    o_ref, l_ref = oracle_dilated(w, inp)
    compare(w, out, lse, o_ref, l_ref, tag=name)


# --------------------------------------------------------------------------
# per-instance segment masks (packed documents): all rows compared
# --------------------------------------------------------------------------
def _seg_case(name, B, H, N, R, G, seg_rows, dtype="bf16", causal=False, dil=None, rel=None,
              sep=False):
    kind, rk = ("scalar", 0) if rel is None else (rel[1], rel[0])
    w = W.Workload(name, B=B, H=H, N=N, dtype=dtype, radius=R, global_idx=G, dilation=dil,
                   causal=causal, rel_k=rk, rel_kind=kind, separate_global=sep, seed=79)
    return w, torch.tensor(np.stack(seg_rows), dtype=torch.int32)


SEG_CASES = [
    # documents of different lengths per batch row, each with its own global tokens
    lambda: _seg_case("seg-packed", 2, 3, 700, 40, (0, 1, 300, 301, 650),
                      [np.repeat([0, 1, 2], [300, 350, 50]), np.repeat([0, 1], [200, 500])]),
    # ETC layout: each document's global tokens first, then the long tokens; label vectors
    lambda: _seg_case("seg-etc-relvec", 1, 2, 32 + 600, 20, tuple(range(32)),
                      [np.concatenate([np.repeat([0, 1], 16), np.repeat([0, 1], [250, 350])])],
                      rel=(6, "both")),
    # ids that are not runs, fp32, causal, per-head dilation (gathered global columns)
    lambda: _seg_case("seg-interleaved-f32", 2, 2, 300, 25, (5, 100, 299),
                      [(np.arange(300) // 37) % 3, (np.arange(300) // 11) % 2], dtype="f32",
                      causal=True, dil=(1, 2)),
    # separate global projections, one document holding everything but a short tail
    lambda: _seg_case("seg-sep-tail", 1, 2, 513, 64, tuple(range(70)),
                      [np.repeat([4, 9], [500, 13])], sep=True),
]


@pytest.mark.parametrize("mk", SEG_CASES, ids=[f"seg{i}" for i in range(len(SEG_CASES))])
def test_segments(dev, mk):
    w, seg = mk()
    inp = W.make_inputs(w)
    inp.seg = seg
    say(f"case {w.name}: B={w.B} H={w.H} N={w.N} R={w.radius} |G|={len(w.global_idx)}")
    out, lse = gpu_attn(w, inp, dev)
    o_ref, l_ref = oracle_attn(w, inp)
    compare(w, out, lse, o_ref, l_ref, tag=w.name)


# --------------------------------------------------------------------------
# Sparse Transformer fixed pattern: all rows compared
# --------------------------------------------------------------------------
FIXED_CASES = [
    # name, B, N, H, (l, c), causal
    ("fixed-heads-wrap", 1, 512, 4, (128, 64), True),     # 4 heads over 2 sub-blocks
    ("fixed-noncausal", 2, 384, 3, (128, 64), False),
    ("fixed-c-equals-l", 1, 256, 2, (128, 128), True),    # dense causal attention
    ("fixed-long-blocks", 1, 1024, 5, (512, 128), True),  # several query tiles per block
    ("fixed-one-block", 1, 256, 2, (256, 64), False),     # no other block: local part only
]


@pytest.mark.parametrize("case", FIXED_CASES, ids=[c[0] for c in FIXED_CASES])
def test_fixed_pattern(dev, case):
    name, B, N, H, lc, causal = case
    w = W.Workload(name, B=B, H=H, N=N, kind="fixed", causal=causal, fixed=lc, seed=81)
    inp = W.make_inputs(w)
    say(f"case {name}: B={B} N={N} H={H} (l, c)={lc} causal={causal}")
    out, lse = gpu_fixed(w, inp, dev)
    o_ref, l_ref = oracle_fixed(w, inp)
    compare(w, out, lse, o_ref, l_ref, tag=name)


# --------------------------------------------------------------------------
# exact mask and global-index handling (Q = 0, V = one-hot(j mod 64))
# --------------------------------------------------------------------------
def _mask_inputs(w, dev):
    B, H, N, D = w.B, w.H, w.N, w.D
    dt = w.torch_dtype
    q = torch.zeros(B, H, N, D, dtype=dt)
    k = torch.randn(B, H, N, D, generator=torch.Generator().manual_seed(5)).to(dt)
    v = torch.zeros(B, H, N, D, dtype=dt)
    v[:, :, torch.arange(N), torch.arange(N) % D] = 1
    sep = None
    if w.separate_global:
        sep = (torch.zeros_like(q), k.flip(2).contiguous(), v.clone())
    return W.Inputs(q, k, v, *(sep or (None, None, None)))


MASK_CASES = [
    W.Workload("mask-longformer", B=1, H=2, N=1000, radius=100, global_idx=(0, 1, 2, 500, 999),
               separate_global=True),
    W.Workload("mask-dilated-causal", B=1, H=3, N=777, radius=40, dilation=(1, 2, 4), causal=True,
               global_idx=(3, 400)),
    W.Workload("mask-f32", B=1, H=1, N=300, dtype="f32", radius=31, global_idx=(150,)),
    W.Workload("mask-etc", B=1, H=2, N=256 + 700, radius=84, global_idx=tuple(range(256))),
]


def _counts(mask):
    cnt = mask.sum(axis=1).astype(np.int64)
    N = mask.shape[1]
    res = np.stack([mask[:, c::64].sum(axis=1) for c in range(64)], axis=1).astype(np.int64)
    return cnt, res


@pytest.mark.parametrize("w", MASK_CASES, ids=[w.name for w in MASK_CASES])
def test_mask_exact(dev, w):
    say(f"case {w.name}")
    inp = _mask_inputs(w, dev)
    out, lse = gpu_attn(w, inp, dev)
    o = to64(out)
    l = to64(lse)
    for h in range(w.H):
        d = w.dilation[h] if w.dilation else 1
        m = oracle.mask_rows(w.N, w.global_idx, w.radius, d, w.causal)
        cnt, res = _counts(m)
        got_cnt = np.rint(np.exp(l[0, h])).astype(np.int64)
        assert np.array_equal(got_cnt, cnt), f"{w.name} h={h}: key counts differ"
        got_res = np.rint(o[0, h] * cnt[:, None]).astype(np.int64)
        assert np.array_equal(got_res, res), f"{w.name} h={h}: allowed key sets differ"


def test_mask_exact_longnet(dev):
    w = W.Workload("mask-longnet", B=1, H=6, N=700, kind="dilated", causal=True,
                   pairs=((64, 1), (128, 2), (256, 4), (700, 6)))
    inp = _mask_inputs(w, dev)
    out, lse = gpu_dilated(w, inp, dev)
    o, l = to64(out), to64(lse)
    for h in range(w.H):
        m = oracle.longnet_mult_rows(w.N, h, w.pairs, True)
        cnt, res = _counts(m)
        assert np.array_equal(np.rint(np.exp(l[0, h])).astype(np.int64), cnt), f"h={h}"
        assert np.array_equal(np.rint(o[0, h] * cnt[:, None]).astype(np.int64), res), f"h={h}"


def _mask_compare(tag, out, lse, o_ref, l_ref):
    """Exact comparison of allowed-key counts and key residues (Q = 0, one-hot V):
    the GPU's rint(exp(lse)) and rint(O * count) against the oracle's."""
    cnt_ref = np.rint(np.exp(l_ref)).astype(np.int64)
    cnt = np.rint(np.exp(to64(lse))).astype(np.int64)
    assert np.array_equal(cnt, cnt_ref), f"{tag}: key counts differ"
    res_ref = np.rint(o_ref * cnt_ref[..., None]).astype(np.int64)
    res = np.rint(to64(out) * cnt_ref[..., None]).astype(np.int64)
    assert np.array_equal(res, res_ref), f"{tag}: allowed key sets differ"


FIXED_MASK_CASES = [
    W.Workload("mask-fixed-causal", B=1, H=5, N=1024, kind="fixed", causal=True, fixed=(256, 64)),
    W.Workload("mask-fixed-full", B=1, H=3, N=768, kind="fixed", causal=False, fixed=(256, 128)),
]


@pytest.mark.parametrize("w", FIXED_MASK_CASES, ids=[w.name for w in FIXED_MASK_CASES])
def test_mask_exact_fixed(dev, w):
    say(f"case {w.name}")
    inp = _mask_inputs(w, dev)
    out, lse = gpu_fixed(w, inp, dev)
    o_ref, l_ref = oracle_fixed(w, inp)
    _mask_compare(w.name, out, lse, o_ref, l_ref)


def test_mask_exact_segments(dev):
    # packed documents of different lengths per batch row, globals in several
    # documents, a dilated head and a causal window: every row's key set
    w = W.Workload("mask-segments", B=2, H=2, N=900, radius=60, dilation=(1, 3), causal=False,
                   global_idx=(0, 1, 300, 301, 640, 899))
    inp = _mask_inputs(w, dev)
    inp.seg = torch.tensor(np.stack([np.repeat([0, 1, 2], [300, 340, 260]),
                                     np.repeat([5, 6], [640, 260])]), dtype=torch.int32)
    say(f"case {w.name}")
    out, lse = gpu_attn(w, inp, dev)
    o_ref, l_ref = oracle_attn(w, inp)
    _mask_compare(w.name, out, lse, o_ref, l_ref)
    wc = w.with_(name="mask-segments-causal", causal=True)
    out, lse = gpu_attn(wc, inp, dev)
    o_ref, l_ref = oracle_attn(wc, inp)
    _mask_compare(wc.name, out, lse, o_ref, l_ref)


# --------------------------------------------------------------------------
# the workloads at full size, in the launch configuration the bench times
# --------------------------------------------------------------------------
def _sel_rows(w, n):
    """Tile edges (every 64th position and its neighbours), edges of the
    sequence, random rows, and every global row of two heads."""
    must = set()
    for t in range(0, w.N, 64):
        must |= {t - 1, t, t + 1}
    must = sorted(i for i in must if 0 <= i < w.N)
    rows = W.sample_rows(w, n, seed=11, must_include=must).numpy()
    if w.global_idx:  # every global row of two heads (the separate pass)
        g = np.array(w.global_idx)
        for (b, h) in ((0, 0), (w.B - 1, w.H - 1)):
            rows = np.concatenate([rows, np.stack([np.full_like(g, b), np.full_like(g, h), g], 1)])
    return rows.astype(np.int32)


# heads with distinct offsets under every pattern of the 32K workloads
# (h mod r for r = 2, 4, 6, 12; summary sub-block h mod 16)
HEADS_32K = (0, 5, 11)


@pytest.mark.parametrize("w", W.ORDERED, ids=[w.name for w in W.ORDERED])
def test_workload_parity(dev, w):
    say(f"workload {w.name}: B={w.B} H={w.H} N={w.N} {w.dtype}")
    inp = W.make_inputs(w)
    if w.kind in ("dilated", "fixed"):
        out, lse = gpu_dilated(w, inp, dev) if w.kind == "dilated" else gpu_fixed(w, inp, dev)
        # every row of three heads
        sel = np.array([(b, h, i) for b in range(w.B) for h in HEADS_32K for i in range(w.N)],
                       dtype=np.int32)
        ref = oracle_dilated if w.kind == "dilated" else oracle_fixed
        o_ref, l_ref = ref(w, inp, sel)
        compare(w, out, lse, o_ref, l_ref, sel, tag=w.name)
        return
    out, lse = gpu_attn(w, inp, dev)
    o_ref, l_ref = oracle_attn(w, inp)  # every row
    compare(w, out, lse, o_ref, l_ref, tag=w.name)


# --------------------------------------------------------------------------
# limits: the largest head count, label clip and pattern count the library
# takes, a long band, many scattered global tokens, a reused workspace
# --------------------------------------------------------------------------
def test_limits_heads_and_labels(dev):
    # H = 64 (per-head dilations 1..4), rel_k = 31 with scalar table and vectors
    w = W.Workload("limits-h64-k31", B=1, H=64, N=300, radius=23, dilation=tuple(1 + h % 4 for h in range(64)),
                   global_idx=(0, 7, 150, 299), rel_k=31, rel_kind="both", seed=91)
    inp = W.make_inputs(w)
    say(f"case {w.name}")
    out, lse = gpu_attn(w, inp, dev)
    o_ref, l_ref = oracle_attn(w, inp)
    compare(w, out, lse, o_ref, l_ref, tag=w.name)


def test_limits_sixteen_patterns(dev):
    pairs = tuple((64 * (1 + p % 4) * (1 + p // 8), 1 + p % 5) for p in range(16))
    w = W.Workload("limits-16-pairs", B=1, H=5, N=1000, kind="dilated", causal=True, pairs=pairs,
                   seed=92)
    inp = W.make_inputs(w)
    say(f"case {w.name}: pairs={pairs}")
    out, lse = gpu_dilated(w, inp, dev)
    o_ref, l_ref = oracle_dilated(w, inp)
    compare(w, out, lse, o_ref, l_ref, tag=w.name)


def test_limits_long_band(dev):
    w = W.Workload("limits-n131072", B=1, H=1, N=131072, radius=512, global_idx=(0, 1, 65536, 131071),
                   seed=93)
    inp = W.make_inputs(w)
    say(f"case {w.name}")
    out, lse = gpu_attn(w, inp, dev)
    sel = _sel_rows(w, 800)
    o_ref, l_ref = oracle_attn(w, inp, sel)
    compare(w, out, lse, o_ref, l_ref, sel, tag=w.name)


def test_limits_many_scattered_globals(dev):
    g = tuple(sorted(set(range(0, 4096, 5)) | {4095}))  # 820 global tokens: gathered columns
    w = W.Workload("limits-820-globals", B=1, H=2, N=4096, radius=100, dilation=(1, 3),
                   global_idx=g, separate_global=True, seed=94)
    inp = W.make_inputs(w)
    say(f"case {w.name}: |G|={len(g)}")
    out, lse = gpu_attn(w, inp, dev)
    sel = _sel_rows(w, 600)
    o_ref, l_ref = oracle_attn(w, inp, sel)
    compare(w, out, lse, o_ref, l_ref, sel, tag=w.name)


def test_workspace_reuse(dev):
    # One workspace, never zero-filled, serves calls of several shapes in turn:
    # its initial contents are arbitrary bytes, and every call leaves partials
    # and counter words where a call of another shape keeps its own. Each
    # call's result must not depend on any of it.
    wa = W.Workload("reuse-a", B=2, H=3, N=1500, radius=60, global_idx=tuple(range(0, 1500, 7)),
                    seed=95)
    wb = W.Workload("reuse-b", B=1, H=2, N=700, radius=30, global_idx=(3, 4, 5, 600), seed=96)
    nb = max(la.la_attn_workspace_size(la.LaDims(w.B, w.H, w.N, 64, la.LA_BF16), len(w.global_idx))
             for w in (wa, wb))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    for x, fill in enumerate(("ones", "random", None, None, None, None)):
        w = (wa, wa, wb, wb, wa, wb)[x]
        if fill == "ones":
            ws.fill_(0xFF)
        elif fill == "random":
            ws.copy_(torch.randint(0, 256, (nb,), dtype=torch.uint8,
                                   generator=torch.Generator().manual_seed(x)).to(dev))
        inp = W.make_inputs(w)
        say(f"case {w.name} (shared workspace, fill={fill})")
        out, lse = gpu_attn(w, inp, dev, workspace=ws)
        o_ref, l_ref = oracle_attn(w, inp)
        compare(w, out, lse, o_ref, l_ref, tag=w.name)
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# determinism, streams, graph capture
# --------------------------------------------------------------------------
def test_deterministic(dev):
    w = W.LONGFORMER_BASE
    inp = W.make_inputs(w)
    a = [gpu_attn(w, inp, dev) for _ in range(3)]
    for o, l in a[1:]:
        assert torch.equal(o, a[0][0]) and torch.equal(l, a[0][1])
    w5 = W.Workload("det-longnet", B=1, H=4, N=4096, kind="dilated", causal=True,
                    pairs=((512, 1), (1024, 2), (4096, 8)))
    inp5 = W.make_inputs(w5)
    b = [gpu_dilated(w5, inp5, dev) for _ in range(3)]
    for o, l in b[1:]:
        assert torch.equal(o, b[0][0]) and torch.equal(l, b[0][1])


def test_nondefault_stream(dev):
    w = W.Workload("stream", B=1, H=2, N=1024, radius=64, global_idx=(0, 10), seed=3)
    inp = W.make_inputs(w)
    ref, _ = gpu_attn(w, inp, dev)
    s = torch.cuda.Stream()
    g = torch.tensor(w.global_idx, dtype=torch.int32, device=dev)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out, _ = la.la_attn_forward(q, k, v, g, w.radius, stream=s)
    s.synchronize()
    assert torch.equal(out, ref)


def test_graph_capture(dev):
    w = W.Workload("graph", B=1, H=2, N=2048, radius=128, global_idx=tuple(range(16)), seed=4)
    inp = W.make_inputs(w)
    g = torch.tensor(w.global_idx, dtype=torch.int32, device=dev)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    ref, ref_lse = la.la_attn_forward(q, k, v, g, w.radius)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = torch.zeros(la.la_attn_workspace_size(la.LaDims(1, 2, 2048, 64, la.LA_BF16), 16),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            la.la_attn_forward(q, k, v, g, w.radius, out=out, lse=lse, workspace=ws, stream=s)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), f"replay {rep}"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays


def test_graph_capture_dilated_and_fixed(dev):
    # the two-launch calls (pattern partials, then the finisher) replay in a graph
    w = W.Workload("graph-longnet", B=1, H=3, N=1024, kind="dilated", causal=True,
                   pairs=((256, 1), (512, 2), (1024, 4)), seed=6)
    inp = W.make_inputs(w)
    q, k, v = inp.q.to(dev), inp.k.to(dev), inp.v.to(dev)
    seg, dil = [p[0] for p in w.pairs], [p[1] for p in w.pairs]
    ref, ref_lse = la.la_dilated_forward(q, k, v, seg, dil, True)
    ref_f, ref_flse = la.la_fixed_forward(q, k, v, 256, 64, True)
    dims = la.LaDims(1, 3, 1024, 64, la.LA_BF16)
    out, out_f = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    lse_f = torch.empty_like(lse)
    ws = torch.empty(la.la_dilated_workspace_size(dims, seg, dil), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(la.la_fixed_workspace_size(dims, 256, 64), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            la.la_dilated_forward(q, k, v, seg, dil, True, out=out, lse=lse, workspace=ws, stream=s)
            la.la_fixed_forward(q, k, v, 256, 64, True, out=out_f, lse=lse_f, workspace=ws_f,
                                stream=s)
    for rep in range(3):
        out.fill_(float("nan"))
        out_f.fill_(float("nan"))
        lse.zero_()
        lse_f.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, ref_lse), f"dilated replay {rep}"
        assert torch.equal(out_f, ref_f) and torch.equal(lse_f, ref_flse), f"fixed replay {rep}"

