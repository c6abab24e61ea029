"""The allocation-free entry point (la_attn_forward_noalloc) against la_attn_forward.

la_attn_forward_noalloc runs the same kernels with the library's fixed device
scratch in place of a caller workspace, so its results must equal
la_attn_forward's bit for bit; both are also held to the oracle's bar. Two
calls follow each other on the shared scratch, the second with a smaller input
(fewer heads, a shorter sequence, other global tokens), so the second call runs
on whatever the first left in the scratch.
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    la.lib()
    return torch.device("cuda:0")


def to64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


CALLS = [
    W.Workload("noalloc-first", B=2, H=4, N=3000, radius=100, global_idx=tuple(range(0, 3000, 9)),
               separate_global=True, seed=501),
    W.Workload("noalloc-second-smaller", B=1, H=2, N=1100, radius=40, global_idx=(0, 7, 500, 1099),
               dilation=(1, 2), seed=502),
]


def test_noalloc_matches_la_attn_forward(dev):
    for w in CALLS:
        print(f"case {w.name}: B={w.B} H={w.H} N={w.N} |G|={len(w.global_idx)}", file=sys.stderr,
              flush=True)
        inp = W.make_inputs(w)
        d = lambda t: None if t is None else t.to(dev)
        g = torch.tensor(w.global_idx, dtype=torch.int32, device=dev)
        args = (d(inp.q), d(inp.k), d(inp.v), g, w.radius, w.dilation, w.causal)
        kw = dict(qg=d(inp.qg), kg=d(inp.kg), vg=d(inp.vg))
        out_n, lse_n = la.la_attn_forward_noalloc(*args, **kw)
        torch.cuda.synchronize()
        out_r, lse_r = la.la_attn_forward(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out_n, out_r), f"{w.name}: out differs from la_attn_forward"
        assert torch.equal(lse_n, lse_r), f"{w.name}: lse differs from la_attn_forward"
        o_ref, l_ref = oracle.attn_rows(to64(inp.q), to64(inp.k), to64(inp.v), w.global_idx,
                                        w.radius, w.dilation, w.causal, None, to64(inp.qg),
                                        to64(inp.kg), to64(inp.vg))
        err = float(np.abs(to64(out_n) - o_ref).max())
        lerr = float(np.abs(to64(lse_n) - l_ref).max())
        assert err <= 2e-2 and lerr <= 2.0 ** -8 + 1e-4, (w.name, err, lerr)


def test_noalloc_rejects_oversized_and_workspace(dev):
    # a call needing more than the 32 MiB scratch is refused before any launch
    q = torch.zeros(4, 16, 8192, 64, dtype=torch.bfloat16, device=dev)
    g = torch.arange(0, 8192, 8, dtype=torch.int32, device=dev)
    with pytest.raises(la.LaError) as e:
        la.la_attn_forward_noalloc(q, q, q, g, 16)
    assert e.value.status == la.LA_EUNSUPPORTED
    with pytest.raises(la.LaError):
        la.bind_attn(q, q, q, g, 16, workspace=torch.empty(16, dtype=torch.uint8, device=dev),
                     noalloc=True)
