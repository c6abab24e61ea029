"""TEST INFRASTRUCTURE — the fp64 CPU oracle for sparse long-sequence attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. The product path (``sparse_long_sequence_amd``)
never imports it, and this package imports nothing from the product: the two
share no code. The arithmetic lives in ``oracle.cpp`` (plain C++17, fp64); this
module only builds it with g++ and marshals numpy arrays through ctypes.

Functions and the passages they follow (details in ``oracle.cpp``):

* :func:`attn_rows` — masked dense softmax attention over the band + global
  pattern (Longformer page §3.4 "Sliding Window Attention", "Dilated Sliding
  Window Attention", "Global Attention", "Separate Linear Projections";
  ETC page §3.4 "Global-Local Attention" and "Relative Position Encoding").
* :func:`mask_rows` — the explicit 0/1 mask rows of that pattern.
* :func:`longnet_rows` — LongNet's mixture as one softmax over the key
  multiplicity (LongNet page §3.4 "Mixture of Dilated Attentions",
  equivalence statement).
* :func:`longnet_mixture_rows` — the same mixture in the page's own order:
  sparsify, attend, scatter, weight by softmax denominators (Eqs. 3-10, 13-15).
* :func:`longnet_mult_rows` — the integer key multiplicity rows.
* :func:`longnet_backward_sel` — the LongNet mixture's gradients for chosen
  rows (dq) and keys (dk, dv), each row evaluated in full by the definition.
* :func:`fixed_rows` — Sparse Transformer's fixed pattern (local block plus
  strided summary positions; LongNet page §3.4 "Standard Self-Attention and
  Sparse Attention (Preliminaries)"), masked dense softmax.

Parity status: every function is pinned by tests in ``tests/test_oracle_pins.py``
(closed-form counts, library special cases, the page's worked index example,
brute force on tiny inputs, and cross-path identities).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib: Optional[ctypes.CDLL] = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def build(src: str = _SRC, out: str = _LIB_PATH, strict: bool = True) -> str:
    """Compile the oracle with g++ (host only) into ``out``."""
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", "-Wall"]
    cmd += ["-Werror"] if strict else ["-w"]
    cmd += [src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = _LIB_PATH) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library at ``path``."""
    global _lib
    if path == _LIB_PATH and _lib is not None:
        return _lib
    if not os.path.exists(path):
        if path != _LIB_PATH:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    lib.lo_version.restype = ctypes.c_int32
    lib.lo_mask_rows.restype = ctypes.c_int32
    lib.lo_mask_rows.argtypes = [ctypes.c_int32, _i32p, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int32, _u8p]
    lib.lo_longnet_mult_rows.restype = ctypes.c_int32
    lib.lo_longnet_mult_rows.argtypes = [ctypes.c_int32, ctypes.c_int32, _i32p, _i32p,
                                         ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int32, _i32p]
    lib.lo_attn_rows.restype = ctypes.c_int32
    lib.lo_attn_rows.argtypes = [ctypes.c_int32] * 4 + [_f64p] * 6 + [
        _i32p, ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int32, _f64p, _f64p,
        ctypes.c_int32, _i32p, _i32p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int32,
        _u8p, _u8p, ctypes.c_int32, ctypes.c_int32]
    lib.lo_fixed_rows.restype = ctypes.c_int32
    lib.lo_fixed_rows.argtypes = [ctypes.c_int32] * 4 + [_f64p] * 3 + [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int64, _f64p, _f64p,
        ctypes.c_int32]
    lib.lo_longnet_rows.restype = ctypes.c_int32
    lib.lo_longnet_rows.argtypes = [ctypes.c_int32] * 4 + [_f64p] * 3 + [
        _i32p, _i32p, ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int64, _f64p, _f64p,
        ctypes.c_int32]
    lib.lo_longnet_mixture_rows.restype = ctypes.c_int32
    lib.lo_longnet_mixture_rows.argtypes = [ctypes.c_int32] * 4 + [_f64p] * 3 + [
        _i32p, _i32p, ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int64, _f64p, _f64p,
        _f64p, _f64p, ctypes.c_int32]
    lib.lo_longnet_backward.restype = ctypes.c_int32
    lib.lo_longnet_backward.argtypes = [ctypes.c_int32] * 4 + [_f64p] * 3 + [
        _i32p, _i32p, ctypes.c_int32, ctypes.c_int32] + [_f64p] * 4 + [ctypes.c_int32]
    lib.lo_longnet_backward_sel.restype = ctypes.c_int32
    lib.lo_longnet_backward_sel.argtypes = [ctypes.c_int32] * 4 + [_f64p] * 3 + [
        _i32p, _i32p, ctypes.c_int32, ctypes.c_int32, _f64p, _i32p, ctypes.c_int64, _f64p,
        _i32p, ctypes.c_int64, _f64p, _f64p, ctypes.c_int32]
    lib.lo_attn_backward.restype = ctypes.c_int32
    lib.lo_attn_backward.argtypes = [ctypes.c_int32] * 4 + [_f64p] * 6 + [
        _i32p, ctypes.c_int32, ctypes.c_int32, _i32p, ctypes.c_int32, _i32p] + [_f64p] * 7 + [
        ctypes.c_int32, _f64p, _f64p, ctypes.c_int32, _u8p, _u8p, ctypes.c_int32, ctypes.c_int32]
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a: Optional[np.ndarray], t):
    return None if a is None else a.ctypes.data_as(t)


def _sel(sel, B, H, N):
    if sel is None:
        return None, B * H * N
    s = _i32(sel).reshape(-1, 3)
    if s.size and ((s[:, 0] < 0).any() or (s[:, 0] >= B).any() or (s[:, 1] < 0).any()
                   or (s[:, 1] >= H).any() or (s[:, 2] < 0).any() or (s[:, 2] >= N).any()):
        raise ValueError("row selection out of range")
    return s, s.shape[0]


def mask_rows(N: int, global_idx: Sequence[int], radius: int, dilation: int = 1,
              causal: bool = False, rows: Optional[Sequence[int]] = None, lib=None) -> np.ndarray:
    """Explicit 0/1 mask rows ``[len(rows) or N, N]`` (uint8) for one head."""
    lib = lib or load()
    g = _i32(sorted(global_idx))
    r = None if rows is None else _i32(rows)
    nr = N if r is None else r.shape[0]
    m = np.zeros((nr, N), dtype=np.uint8)
    rc = lib.lo_mask_rows(N, _p(g, _i32p), g.shape[0], radius, dilation, int(causal),
                          _p(r, _i32p), nr, _p(m, _u8p))
    if rc != 0:
        raise ValueError("lo_mask_rows rejected its arguments")
    return m


def longnet_mult_rows(N: int, head: int, pairs: Sequence[Sequence[int]], causal: bool = True,
                      rows: Optional[Sequence[int]] = None, lib=None) -> np.ndarray:
    """Integer key multiplicity rows ``[len(rows) or N, N]`` (int32) for one head."""
    lib = lib or load()
    w = _i32([p[0] for p in pairs])
    rr = _i32([p[1] for p in pairs])
    r = None if rows is None else _i32(rows)
    nr = N if r is None else r.shape[0]
    m = np.zeros((nr, N), dtype=np.int32)
    rc = lib.lo_longnet_mult_rows(N, head, _p(w, _i32p), _p(rr, _i32p), w.shape[0], int(causal),
                                  _p(r, _i32p), nr, _p(m, _i32p))
    if rc != 0:
        raise ValueError("lo_longnet_mult_rows rejected its arguments")
    return m


LABEL_DISTANCE = 0xFE  # a pair's usual clipped-distance label
LABEL_MASKED = 0xFF    # any value >= the vocabulary size (but LABEL_DISTANCE) masks the pair


def _labels(rel_bias, rel_vec, rel_k, glabel, llabel, B, H, N, D, n_global):
    """Checked bias tables and label matrices: (rel_bias, rel_vec, rel_k,
    n_labels, glabel, llabel) in the library's types (n_labels 0: no table)."""
    rb = None if rel_bias is None else _f64(rel_bias)
    rv = None if rel_vec is None else _f64(rel_vec)
    V = None
    if rb is not None:
        if rb.ndim != 2 or rb.shape[0] != H:
            raise ValueError("rel_bias must be [H, V]")
        V = rb.shape[1]
    if rv is not None:
        if rv.ndim != 3 or rv.shape[0] != H or rv.shape[2] != D:
            raise ValueError("rel_vec must be [H, V, D]")
        if V is not None and rv.shape[1] != V:
            raise ValueError("rel_bias and rel_vec need the same vocabulary")
        V = rv.shape[1]
    rk = 0
    if V is not None:
        if rel_k is None:
            if V % 2 != 1:
                raise ValueError("give rel_k with a vocabulary of structural labels")
            rel_k = (V - 1) // 2
        rk = int(rel_k)
        if V < 2 * rk + 1:
            raise ValueError("the vocabulary holds fewer than 2k+1 labels")
    gl = ll = None
    if glabel is not None:
        gl = np.ascontiguousarray(np.asarray(glabel, dtype=np.uint8))
        if gl.shape != (B, n_global, N):
            raise ValueError("glabel must be [B, n_global, N]")
    if llabel is not None:
        ll = np.ascontiguousarray(np.asarray(llabel, dtype=np.uint8))
        if ll.shape != (B, N, n_global):
            raise ValueError("llabel must be [B, N, n_global]")
    return rb, rv, rk, 0 if V is None else V, gl, ll


def attn_rows(q, k, v, global_idx=(), radius: int = 0, dilation=None, causal: bool = False,
              rel_bias=None, qg=None, kg=None, vg=None, sel=None, n_threads: int = 0, lib=None,
              rel_vec=None, seg=None, rel_k=None, glabel=None, llabel=None, seg_pieces: int = 0):
    """Band + global attention in fp64.

    ``q, k, v`` (and optional ``qg, kg, vg``) are ``[B,H,N,D]``. ``dilation`` is
    per head (``None`` = all 1). ``rel_bias`` is ``[H, V]`` (a scalar per
    label) and ``rel_vec`` ``[H, V, D]`` (a key-side vector per label); either,
    both or neither may be given. The vocabulary is the 2k+1 clipped-distance
    labels (``V = 2k+1``, k from the table's width unless ``rel_k`` is given),
    followed by ``V - 2k - 1`` structural labels. ``seg`` (``[B,N]`` int)
    gives each token a segment id: pairs across segments are masked in the
    pieces ``seg_pieces`` selects (bits g2g 1, g2l 2, l2g 4, l2l 8; 0 = all).
    ``glabel`` (``[B, n_global, N]`` uint8) labels the pairs of each global query
    (g2g, g2l) and ``llabel`` (``[B, N, n_global]`` uint8) the pairs of a non-global
    query with each global key (l2g): a vocabulary index, ``LABEL_DISTANCE``, or
    a masked pair (any other value). ``sel`` is an ``[n,3]`` array of ``(b,h,i)``
    rows (``None`` = all rows). Returns ``(out [n,D], lse [n])`` as float64; with
    ``sel=None`` they are reshaped to ``[B,H,N,D]`` and ``[B,H,N]``.
    """
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    sep = [x is not None for x in (qg, kg, vg)]
    if any(sep) and not all(sep):
        raise ValueError("qg, kg, vg must be given together")
    qg, kg, vg = [None if x is None else _f64(x) for x in (qg, kg, vg)]
    for x in (qg, kg, vg):
        if x is not None and x.shape != q.shape:
            raise ValueError("global projection shape differs from q")
    g = _i32(sorted(global_idx))
    dil = None if dilation is None else _i32(dilation)
    if dil is not None and dil.shape != (H,):
        raise ValueError("dilation must have one entry per head")
    rb, rv, rk, nlab, gl, ll = _labels(rel_bias, rel_vec, rel_k, glabel, llabel, B, H, N, D,
                                       g.shape[0])
    sg = None
    if seg is not None:
        sg = _i32(seg)
        if sg.shape != (B, N):
            raise ValueError("seg must be [B, N]")
    s, n = _sel(sel, B, H, N)
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = lib.lo_attn_rows(B, H, N, D, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p), _p(qg, _f64p),
                          _p(kg, _f64p), _p(vg, _f64p), _p(g, _i32p), g.shape[0], radius,
                          _p(dil, _i32p), int(causal), _p(rb, _f64p), _p(rv, _f64p), rk,
                          _p(sg, _i32p), _p(s, _i32p), n,
                          _p(out, _f64p), _p(lse, _f64p), n_threads, _p(gl, _u8p), _p(ll, _u8p),
                          nlab, int(seg_pieces))
    if rc != 0:
        raise ValueError("lo_attn_rows rejected its arguments")
    if sel is None:
        return out.reshape(B, H, N, D), lse.reshape(B, H, N)
    return out, lse


def attn_backward(q, k, v, dout, global_idx=(), radius: int = 0, dilation=None,
                  causal: bool = False, qg=None, kg=None, vg=None, seg=None, n_threads: int = 0,
                  lib=None, rel_bias=None, rel_vec=None, rel_k=None, glabel=None, llabel=None,
                  seg_pieces: int = 0):
    """Gradients of band + global attention in fp64 for upstream gradient ``dout``.

    Arguments as in :func:`attn_rows` (the bias tables are inputs, not
    differentiated). Returns ``(dq, dk, dv)``, or ``(dq, dk, dv, dqg, dkg,
    dvg)`` with separate global projections, each ``[B,H,N,D]`` float64.
    """
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    if k.shape != q.shape or v.shape != q.shape or do.shape != q.shape:
        raise ValueError("q, k, v, dout shapes differ")
    sep = [x is not None for x in (qg, kg, vg)]
    if any(sep) and not all(sep):
        raise ValueError("qg, kg, vg must be given together")
    qg, kg, vg = [None if x is None else _f64(x) for x in (qg, kg, vg)]
    g = _i32(sorted(global_idx))
    dil = None if dilation is None else _i32(dilation)
    if dil is not None and dil.shape != (H,):
        raise ValueError("dilation must have one entry per head")
    sg = None if seg is None else _i32(seg)
    if sg is not None and sg.shape != (B, N):
        raise ValueError("seg must be [B, N]")
    rb, rv, rk, nlab, gl, ll = _labels(rel_bias, rel_vec, rel_k, glabel, llabel, B, H, N, D,
                                       g.shape[0])
    grads = [np.zeros_like(q) for _ in range(6 if all(sep) else 3)]
    ptr = [_p(x, _f64p) for x in grads] + [None] * (6 - len(grads))
    rc = lib.lo_attn_backward(B, H, N, D, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                              _p(qg, _f64p), _p(kg, _f64p), _p(vg, _f64p), _p(g, _i32p),
                              g.shape[0], radius, _p(dil, _i32p), int(causal), _p(sg, _i32p),
                              _p(do, _f64p), *ptr, n_threads, _p(rb, _f64p), _p(rv, _f64p), rk,
                              _p(gl, _u8p), _p(ll, _u8p), nlab, int(seg_pieces))
    if rc != 0:
        raise ValueError("lo_attn_backward rejected its arguments")
    return tuple(grads)


def longnet_backward(q, k, v, dout, pairs, causal: bool = True, n_threads: int = 0, lib=None):
    """Gradients ``(dq, dk, dv)`` of the LongNet mixture in fp64 (``[B,H,N,D]``)."""
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    w, r = _pairs(pairs)
    grads = [np.zeros_like(q) for _ in range(3)]
    rc = lib.lo_longnet_backward(B, H, N, D, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                                 _p(w, _i32p), _p(r, _i32p), w.shape[0], int(causal),
                                 _p(do, _f64p), *[_p(x, _f64p) for x in grads], n_threads)
    if rc != 0:
        raise ValueError("lo_longnet_backward rejected its arguments")
    return tuple(grads)


def longnet_backward_sel(q, k, v, dout, pairs, causal: bool = True, rows=None, keys=None,
                         n_threads: int = 0, lib=None):
    """Chosen LongNet mixture gradients in fp64: ``dq`` of the ``rows`` and ``dk``,
    ``dv`` of the ``keys`` (each an ``[n, 3]`` array of (b, h, position)),
    every row involved evaluated in full. Returns ``(dq [n_rows, D],
    dk [n_keys, D], dv [n_keys, D])``."""
    lib = lib or load()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, N, D = q.shape
    w, r = _pairs(pairs)
    rs, nr = _sel(np.zeros((0, 3)) if rows is None else rows, B, H, N)
    ks, nk = _sel(np.zeros((0, 3)) if keys is None else keys, B, H, N)
    dq = np.zeros((nr, D))
    dk = np.zeros((nk, D))
    dv = np.zeros((nk, D))
    rc = lib.lo_longnet_backward_sel(B, H, N, D, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                                     _p(w, _i32p), _p(r, _i32p), w.shape[0], int(causal),
                                     _p(do, _f64p), _p(rs, _i32p), nr, _p(dq, _f64p),
                                     _p(ks, _i32p), nk, _p(dk, _f64p), _p(dv, _f64p), n_threads)
    if rc != 0:
        raise ValueError("lo_longnet_backward_sel rejected its arguments")
    return dq, dk, dv


def fixed_rows(q, k, v, block_len: int, summary_len: int, causal: bool = True, sel=None,
               n_threads: int = 0, lib=None):
    """Sparse Transformer fixed pattern in fp64 (block length l, c summary
    positions per block; head h takes the sub-block l - c(h'+1) .. l - c h' - 1,
    h' = h mod floor(l/c)). Shapes and returns as :func:`attn_rows`."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    s, n = _sel(sel, B, H, N)
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = lib.lo_fixed_rows(B, H, N, D, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p), int(block_len),
                           int(summary_len), int(causal), _p(s, _i32p), n, _p(out, _f64p),
                           _p(lse, _f64p), n_threads)
    if rc != 0:
        raise ValueError("lo_fixed_rows rejected its arguments")
    if sel is None:
        return out.reshape(B, H, N, D), lse.reshape(B, H, N)
    return out, lse


def _pairs(pairs):
    w = _i32([p[0] for p in pairs])
    r = _i32([p[1] for p in pairs])
    if w.shape[0] < 1:
        raise ValueError("at least one (w, r) pair")
    return w, r


def longnet_rows(q, k, v, pairs, causal: bool = True, sel=None, n_threads: int = 0, lib=None):
    """LongNet mixture via one softmax over the key multiplicity (fp64)."""
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    w, r = _pairs(pairs)
    s, n = _sel(sel, B, H, N)
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    rc = lib.lo_longnet_rows(B, H, N, D, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p), _p(w, _i32p),
                             _p(r, _i32p), w.shape[0], int(causal), _p(s, _i32p), n,
                             _p(out, _f64p), _p(lse, _f64p), n_threads)
    if rc != 0:
        raise ValueError("lo_longnet_rows rejected its arguments")
    if sel is None:
        return out.reshape(B, H, N, D), lse.reshape(B, H, N)
    return out, lse


def longnet_mixture_rows(q, k, v, pairs, causal: bool = True, sel=None, per_pattern: bool = False,
                         n_threads: int = 0, lib=None):
    """LongNet mixture in the page's order (sparsify, attend, scatter, mix).

    With ``per_pattern`` also returns ``(out_k [P,n,D], lse_k [P,n])``.
    """
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    w, r = _pairs(pairs)
    P = w.shape[0]
    s, n = _sel(sel, B, H, N)
    out = np.zeros((n, D), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    ok = np.zeros((P, n, D), dtype=np.float64) if per_pattern else None
    lk = np.zeros((P, n), dtype=np.float64) if per_pattern else None
    rc = lib.lo_longnet_mixture_rows(B, H, N, D, _p(q, _f64p), _p(k, _f64p), _p(v, _f64p),
                                     _p(w, _i32p), _p(r, _i32p), P, int(causal), _p(s, _i32p), n,
                                     _p(out, _f64p), _p(lse, _f64p), _p(ok, _f64p), _p(lk, _f64p),
                                     n_threads)
    if rc != 0:
        raise ValueError("lo_longnet_mixture_rows rejected its arguments")
    if sel is None:
        out, lse = out.reshape(B, H, N, D), lse.reshape(B, H, N)
        if per_pattern:
            ok, lk = ok.reshape(P, B, H, N, D), lk.reshape(P, B, H, N)
    if per_pattern:
        return out, lse, ok, lk
    return out, lse
