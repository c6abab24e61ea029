"""The bench's useful-work count against the oracle's own masks.

`flops.useful_pairs` (4*D FLOPs per allowed pair) is the numerator of every
TFLOP/s figure the bench reports. Here it is checked against the number of
allowed (query, key) pairs the fp64 oracle's mask predicates give, read as
exp(lse) with Q = K = V = 0 (every logit 0, so each row's softmax denominator
is its key count, or multiplicity sum for LongNet), for all nine workloads.
Band workloads are counted over every row (heads with the same pattern are
counted once and multiplied). The two 32K-token workloads are counted over
every row of three heads with distinct offsets; their totals over all heads
are the closed forms pinned in the oracle's pins.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from sparse_long_sequence_amd import flops as F
from sparse_long_sequence_amd import workloads as W

DZ = 4  # head dimension of the zero inputs: the counts do not depend on it


def _band_count(w: W.Workload) -> int:
    """Allowed pairs of a band workload by the oracle, summed over B and H."""
    dils = list(w.dilation) if w.dilation else [1] * w.H
    distinct = sorted(set(dils))
    seg = None
    B = w.B
    if w.documents:
        seg = W.make_inputs(w.with_(B=1, H=1, N=w.N)).seg.numpy()
        B = 1
    z = np.zeros((B, len(distinct), w.N, DZ))
    kw = {}
    if w.structure:  # label matrices and the piece-selected segment ids
        st = W.etc_structure(w.with_(B=1))
        B, seg = 1, st["seg"]
        z = np.zeros((B, len(distinct), w.N, DZ))
        # a zero table of the full vocabulary: structural labels count as allowed
        kw = dict(glabel=st["glabel"], llabel=st["llabel"], seg_pieces=st["seg_pieces"],
                  rel_bias=np.zeros((len(distinct), st["n_labels"])), rel_k=w.rel_k)
    _, lse = oracle.attn_rows(z, z, z, w.global_idx, w.radius, distinct, w.causal, seg=seg, **kw)
    per = {d: int(np.rint(np.exp(lse[:, x])).sum()) for x, d in enumerate(distinct)}
    rows_b = w.B // B
    return rows_b * sum(per[d] for d in dils)


BAND = [w for w in W.ORDERED if w.kind == "band"]


@pytest.mark.parametrize("w", BAND, ids=[w.name for w in BAND])
def test_band_pairs_match_oracle(w):
    if w.documents:  # the same documents in every batch row
        ids = W.make_inputs(w.with_(B=2, H=1)).seg.numpy()
        assert (ids[0] == ids[1]).all()
    assert F.useful_pairs(w) == _band_count(w)


def test_headline_pairs_closed_form():
    assert F.useful_pairs(W.LONGFORMER_BASE) == 60_547_584
    assert F.useful_flops(W.LONGFORMER_BASE) == 15_500_181_504
    assert F.useful_pairs(W.ETC_SHAPE) == 34_173_264


def test_longnet_pairs_match_oracle():
    w = W.LONGNET_SHARE
    assert F.useful_pairs(w) == 839_254_020
    z = np.zeros((1, w.H, w.N, DZ))
    for h in (0, 5, 11):
        sel = np.stack([np.zeros(w.N), np.full(w.N, h), np.arange(w.N)], 1).astype(np.int32)
        _, lse = oracle.longnet_rows(z, z, z, w.pairs, w.causal, sel=sel)
        assert int(np.rint(np.exp(lse)).sum()) == F.dilated_pairs_head(w, h), h


def test_fixed_pairs_match_oracle():
    w = W.FIXED_SHARE
    z = np.zeros((1, w.H, w.N, DZ))
    per_head = F.fixed_pairs(w) // (w.B * w.H)
    assert per_head * w.B * w.H == F.fixed_pairs(w)
    for h in (0, 7):
        sel = np.stack([np.zeros(w.N), np.full(w.N, h), np.arange(w.N)], 1).astype(np.int32)
        _, lse = oracle.fixed_rows(z, z, z, w.fixed[0], w.fixed[1], w.causal, sel=sel)
        assert int(np.rint(np.exp(lse)).sum()) == per_head, h
