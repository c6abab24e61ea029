"""Seeded synthetic workloads for sparse long-sequence attention.

This module holds only workload descriptions (shapes, pattern parameters) and
seeded random inputs. It contains none of the attention arithmetic, so both the
HIP path and the CPU oracle may draw their inputs from it.

The five named workloads stand in for the pages' data (document QA at 4,096
tokens, ETC long inputs with one global summary token per sentence, character
language modelling at 16,384 tokens, LongNet's 32K sequences); no dataset is
read. Recipe: ``torch.Generator('cpu').manual_seed(seed)``; draw order q, k, v,
then qg, kg, vg (when the workload has separate global projections), then the
relative-bias table as 0.1 * N(0,1), then the key-side label vectors as
0.1 * N(0,1); values iid N(0,1) in fp32, then rounded to bf16
(round-to-nearest-even) for bf16 workloads (the bias tables stay fp32).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    """One attention call: shapes, dtype and pattern parameters."""

    name: str
    B: int
    H: int
    N: int
    D: int = 64
    dtype: str = "bf16"                     # "bf16" or "f32"
    kind: str = "band"                      # "band" (la_attn_forward), "dilated" (la_dilated_forward)
                                            # or "fixed" (la_fixed_forward)
    radius: int = 0
    global_idx: Tuple[int, ...] = ()
    dilation: Optional[Tuple[int, ...]] = None  # per head; None = all 1
    causal: bool = False
    rel_k: int = 0                          # >0: relative-position labels clip at k
    rel_kind: str = "scalar"                # with rel_k > 0: "scalar" table [H][2k+1],
                                            # "vector" key-side vectors [H][2k+1][D], or "both"
    separate_global: bool = False
    pairs: Tuple[Tuple[int, int], ...] = ()  # LongNet (segment length w, dilation r)
    fixed: Tuple[int, int] = ()             # fixed pattern: (block length l, summary length c)
    documents: Tuple[int, ...] = ()         # packed documents: lengths in order (segment
                                            # masks; positions past them form one more)
    structure: Tuple[int, int] = ()         # ETC structured input: (contexts, candidates);
                                            # global_idx = range(n_global), see etc_structure
    seed: int = 0

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the hot path. Seeds are 1000 + index.
TINY = Workload("tiny-local-global", B=1, H=1, N=512, dtype="f32", radius=32,
                global_idx=(0, 1), seed=1001)
LONGFORMER_BASE = Workload("longformer-base-n4096-r256-g64", B=2, H=12, N=4096, radius=256,
                           global_idx=tuple(range(64)), separate_global=True, seed=1002)
ETC_SHAPE = Workload("etc-ng256-nl4096-r84-relk12", B=1, H=12, N=256 + 4096, radius=84,
                     global_idx=tuple(range(256)), rel_k=12, seed=1003)
CHARLM_DILATED = Workload("charlm-causal-n16384-w512-dil", B=1, H=8, N=16384, radius=512,
                          dilation=(1, 1, 1, 1, 1, 1, 2, 2), causal=True, seed=1004)
LONGNET_SHARE = Workload("longnet-n32768-5pairs", B=1, H=12, N=32768, kind="dilated", causal=True,
                         pairs=((2048, 1), (4096, 2), (8192, 4), (16384, 6), (32768, 12)),
                         seed=1005)

# ETC's own relative-position mechanism on the same shape: a learned key-side
# vector per label and head instead of the scalar stand-in.
# Sparse Transformer's fixed pattern, LongNet's baseline, on the LongNet shape:
# blocks of 2048 and 128 summary positions per block (the block size the
# LongNet page names; c sets the sparsity, here within 10% of the LongNet
# workload's pairs, as that page matches the two by FLOPs).
FIXED_SHARE = Workload("sparse-transformer-fixed-n32768-l2048-c128", B=1, H=12, N=32768,
                       kind="fixed", causal=True, fixed=(2048, 128), seed=1008)

# Document packing (per-instance segment masks): the Longformer-base shape
# holding four documents of 1024 tokens per sequence, each with its first 16
# tokens global.
PACKED = Workload("longformer-packed-4x1024-g16", B=2, H=12, N=4096, radius=256,
                  global_idx=tuple(d * 1024 + t for d in range(4) for t in range(16)),
                  separate_global=True, documents=(1024, 1024, 1024, 1024), seed=1007)

ETC_VECTORS = Workload("etc-ng256-nl4096-r84-relvec12", B=1, H=12, N=256 + 4096, radius=84,
                       global_idx=tuple(range(256)), rel_k=12, rel_kind="vector", seed=1006)

# ETC's structured input on the same shape: 16 contexts of sentences with one
# global token per sentence and per context, a CLS token and 7 answer
# candidates; per-instance masks and four structural labels (see etc_structure).
ETC_STRUCTURED = Workload("etc-structured-ng256-nl4096-r84-relvec12-v29", B=1, H=12,
                          N=256 + 4096, radius=84, global_idx=tuple(range(256)), rel_k=12,
                          rel_kind="vector", structure=(16, 7), seed=1009)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY, LONGFORMER_BASE, ETC_SHAPE, CHARLM_DILATED, LONGNET_SHARE,
                                   ETC_VECTORS, PACKED, FIXED_SHARE, ETC_STRUCTURED)}
ORDERED: List[Workload] = [TINY, LONGFORMER_BASE, ETC_SHAPE, CHARLM_DILATED, LONGNET_SHARE,
                           ETC_VECTORS, PACKED, FIXED_SHARE, ETC_STRUCTURED]


@dataclass
class Inputs:
    """CPU tensors for one call (dtype as the workload; rel_bias fp32)."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    qg: Optional[torch.Tensor] = None
    kg: Optional[torch.Tensor] = None
    vg: Optional[torch.Tensor] = None
    rel_bias: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)
    rel_vec: Optional[torch.Tensor] = None
    seg: Optional[torch.Tensor] = None      # int32 [B, N] segment ids
    glabel: Optional[torch.Tensor] = None   # uint8 [B, n_global, N] labels of global rows
    llabel: Optional[torch.Tensor] = None   # uint8 [B, N, n_global] labels of l2g pairs
    seg_pieces: int = 0                     # pieces the segment ids mask (0 = all)
    rel_k: Optional[int] = None             # clip distance when the vocabulary is wider


def make_inputs(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw the workload's inputs on the CPU from ``seed`` (default ``w.seed``)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.D)

    def draw(sz):
        return torch.randn(sz, generator=g, dtype=torch.float32)

    q, k, v = draw(shape), draw(shape), draw(shape)
    qg = kg = vg = None
    if w.separate_global:
        qg, kg, vg = draw(shape), draw(shape), draw(shape)
    rb = rv = None
    nv = 2 * w.rel_k + 1 + (N_STRUCT_LABELS if w.structure else 0)
    if w.rel_k > 0 and w.rel_kind in ("scalar", "both"):
        rb = 0.1 * draw((w.H, nv))
    if w.rel_k > 0 and w.rel_kind in ("vector", "both"):
        rv = 0.1 * draw((w.H, nv, w.D))
    dt = w.torch_dtype
    cast = (lambda t: None if t is None else t.to(dt).contiguous())
    seg = None
    if w.documents:
        ids = torch.full((w.N,), len(w.documents), dtype=torch.int32)
        off = 0
        for dn, n in enumerate(w.documents):
            ids[off:off + n] = dn
            off += n
        seg = ids.expand(w.B, w.N).contiguous()
    inp = Inputs(cast(q), cast(k), cast(v), cast(qg), cast(kg), cast(vg),
                 None if rb is None else rb.contiguous(),
                 rel_vec=None if rv is None else rv.contiguous(), seg=seg)
    if w.structure:
        st = etc_structure(w)
        inp.glabel = torch.from_numpy(st["glabel"])
        inp.llabel = torch.from_numpy(st["llabel"])
        inp.seg = torch.from_numpy(st["seg"])
        inp.seg_pieces = st["seg_pieces"]
        inp.rel_k = w.rel_k
    return inp


# Structural labels after the 2k+1 distance labels, and the two special label
# values of the label matrices.
N_STRUCT_LABELS = 4
LABEL_DISTANCE = 0xFE  # the pair keeps its usual clipped-distance label
LABEL_MASKED = 0xFF    # the pair is masked


def etc_structure(w: Workload) -> dict:
    """Seeded structure of an ETC input (ETC page, 3.4 "How Global-Local
    Attention Encodes Structured Inputs" and "Per-instance attention masks").

    The long input (N - n_global word pieces) is cut into ``contexts`` equal
    runs; each context into sentences of random length (at least 4 pieces).
    Global tokens, in order: one CLS, one per context, one per sentence, and
    ``candidates`` answer tokens, each mentioned at 6 random word pieces.
    Masks: a sentence token's g2l attention is hard (its own sentence's pieces
    only), sentence tokens of different contexts do not see each other (g2g),
    and l2l attention stays inside a context (the segment ids, l2l piece only).
    Labels (k = w.rel_k, V = 2k+1+4): 2k+1 "belongs" between a sentence token
    and its pieces (both directions), 2k+2 "does not belong" from a piece to
    the other sentence tokens (l2g), 2k+3 "mention" between a candidate and its
    mentions, 2k+4 "part of" from a sentence token to its context token; every
    other pair keeps its clipped relative-distance label (mixed pairs: none).
    The recipe draws from numpy's default_rng(w.seed + 7); per batch row the
    same structure."""
    import numpy as np

    n_ctx, n_cand = w.structure
    ng = len(w.global_idx)
    nl = w.N - ng
    n_sent = ng - 1 - n_ctx - n_cand
    if w.global_idx != tuple(range(ng)) or n_sent < n_ctx or nl < 4 * n_sent:
        raise ValueError("structure needs the globals first and room for every sentence")
    rng = np.random.default_rng(w.seed + 7)
    # sentences per context (as even as possible), then their lengths
    per_ctx = np.full(n_ctx, n_sent // n_ctx)
    per_ctx[: n_sent % n_ctx] += 1
    ctx_len = np.full(n_ctx, nl // n_ctx)
    ctx_len[: nl % n_ctx] += 1
    sent_of = np.empty(nl, dtype=np.int64)       # word piece -> sentence
    ctx_of_sent = np.repeat(np.arange(n_ctx), per_ctx)
    pos, s0 = 0, 0
    for c in range(n_ctx):
        m = int(per_ctx[c])
        extra = rng.multinomial(int(ctx_len[c]) - 4 * m, np.full(m, 1.0 / m))
        for t, L in enumerate(4 + extra):
            sent_of[pos:pos + L] = s0 + t
            pos += L
        s0 += m
    ctx_of = ctx_of_sent[sent_of]                 # word piece -> context
    mentions = [rng.choice(nl, size=6, replace=False) for _ in range(n_cand)]
    k = w.rel_k
    BEL, NOT, MEN, PART = 2 * k + 1, 2 * k + 2, 2 * k + 3, 2 * k + 4
    g_ctx = 1 + np.arange(n_ctx)                  # global index of context c
    g_sent = 1 + n_ctx + np.arange(n_sent)        # global index of sentence s
    g_cand = 1 + n_ctx + n_sent + np.arange(n_cand)
    N = w.N
    glabel = np.full((ng, N), LABEL_DISTANCE, dtype=np.uint8)
    llabel = np.full((N, ng), LABEL_DISTANCE, dtype=np.uint8)
    longs = ng + np.arange(nl)
    for s in range(n_sent):
        g = g_sent[s]
        own = sent_of == s
        glabel[g, longs] = np.where(own, BEL, LABEL_MASKED)          # hard g2l
        other_ctx = ctx_of_sent != ctx_of_sent[s]
        glabel[g, g_sent[other_ctx]] = LABEL_MASKED                   # cross-context g2g
        glabel[g, g_ctx[ctx_of_sent[s]]] = PART
        llabel[longs, g] = np.where(own, BEL, NOT)
    for c in range(n_cand):
        glabel[g_cand[c], ng + mentions[c]] = MEN
        llabel[ng + mentions[c], g_cand[c]] = MEN
    seg = np.concatenate([np.zeros(ng, dtype=np.int32), 1 + ctx_of.astype(np.int32)])
    B = w.B
    return {"glabel": np.broadcast_to(glabel, (B, ng, N)).copy(),
            "llabel": np.broadcast_to(llabel, (B, N, ng)).copy(),
            "seg": np.broadcast_to(seg, (B, N)).copy(),
            "seg_pieces": 8, "n_labels": 2 * k + 1 + N_STRUCT_LABELS}


def sample_rows(w: Workload, n: int, seed: int = 7, must_include=()) -> torch.Tensor:
    """``[n, 3]`` int32 (b, h, i) rows: edges, pattern boundaries and random rows."""
    g = torch.Generator("cpu").manual_seed(seed)
    rows = []
    edge = sorted({0, 1, w.N - 1, w.N - 2, w.N // 2} | set(i for i in must_include if 0 <= i < w.N))
    for b in range(w.B):
        for h in range(w.H):
            for i in edge:
                rows.append((b, h, i))
    extra = max(0, n - len(rows))
    if extra:
        bb = torch.randint(0, w.B, (extra,), generator=g)
        hh = torch.randint(0, w.H, (extra,), generator=g)
        ii = torch.randint(0, w.N, (extra,), generator=g)
        rows += list(zip(bb.tolist(), hh.tolist(), ii.tolist()))
    return torch.tensor(rows, dtype=torch.int32)
