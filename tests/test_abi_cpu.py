"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/longattn.h declares, sizes its workspaces, and rejects bad
arguments before touching the device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import sparse_long_sequence_amd as la
from sparse_long_sequence_amd import LaAttnExt, LaDilatedExt, LaDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "longattn.h")
FAKE = 0x10000  # a non-null, 256-byte aligned address; never dereferenced by these calls


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(la.LIB_PATH):
        from sparse_long_sequence_amd import build
        build.build()
    return la.lib()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_symbols() == sorted(la.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), name
    assert la.la_version() == 2


def _attn(L, dims, q=FAKE, k=FAKE, v=FAKE, gidx=None, n_global=0, radius=0, dil=None,
          causal=0, rel_bias=None, out=FAKE, lse=None, ext=None):
    return L.la_attn_forward(ctypes.byref(dims) if dims is not None else None, q, k, v, gidx,
                             n_global, radius, dil, causal, rel_bias, out, lse, None,
                             ctypes.byref(ext) if ext is not None else None)


def test_attn_argument_errors(L):
    d = LaDims(1, 2, 128, 64, la.LA_BF16)
    assert _attn(L, None) == la.LA_EINVAL
    assert _attn(L, LaDims(-1, 2, 128, 64, la.LA_BF16)) == la.LA_EINVAL
    assert _attn(L, LaDims(1, 2, 128, 64, 7)) == la.LA_EINVAL
    assert "dtype" in la.la_last_error()
    assert _attn(L, LaDims(1, 2, 128, 32, la.LA_BF16)) == la.LA_EUNSUPPORTED
    assert _attn(L, d, q=None) == la.LA_EINVAL
    assert _attn(L, d, q=FAKE + 2) == la.LA_EINVAL          # misaligned
    assert _attn(L, d, radius=-1) == la.LA_EINVAL
    assert _attn(L, d, causal=2) == la.LA_EINVAL
    assert _attn(L, d, n_global=3) == la.LA_EINVAL           # count without indices
    assert _attn(L, d, gidx=FAKE, n_global=0) == la.LA_EINVAL
    assert _attn(L, d, gidx=FAKE, n_global=129) == la.LA_EINVAL
    bad_dil = (ctypes.c_int32 * 2)(1, 0)
    assert _attn(L, d, dil=bad_dil) == la.LA_EINVAL
    assert _attn(L, d, rel_bias=FAKE) == la.LA_EINVAL        # rel_bias without rel_k
    assert _attn(L, d, ext=LaAttnExt(3, None, None, None, None, 0)) == la.LA_EINVAL
    assert _attn(L, d, rel_bias=FAKE, ext=LaAttnExt(40, None, None, None, None, 0)) == \
        la.LA_EUNSUPPORTED
    assert _attn(L, d, ext=LaAttnExt(0, FAKE, None, None, None, 0)) == la.LA_EINVAL
    # key-side label vectors: need rel_k >= 1 and a 16-byte aligned table
    assert _attn(L, d, ext=LaAttnExt(0, None, None, None, None, 0, FAKE)) == la.LA_EINVAL
    assert _attn(L, d, ext=LaAttnExt(2, None, None, None, None, 0, FAKE + 4)) == la.LA_EINVAL
    # segment ids must be 4-byte aligned
    assert _attn(L, d, ext=LaAttnExt(0, None, None, None, None, 0, None, FAKE + 2)) == la.LA_EINVAL
    # structural labels: vocabulary size, label matrices and piece selection
    E = lambda rk, nl=0, gl=None, ll=None, sp=0: LaAttnExt(rk, None, None, None, None, 0, None,
                                                          None, gl, ll, nl, sp)
    assert _attn(L, d, rel_bias=FAKE, ext=E(2, nl=4)) == la.LA_EINVAL     # below 2k+1
    assert _attn(L, d, rel_bias=FAKE, ext=E(2, nl=65)) == la.LA_EUNSUPPORTED
    assert _attn(L, d, ext=E(0, nl=8)) == la.LA_EINVAL                     # labels, no table
    assert _attn(L, d, ext=E(0, gl=FAKE)) == la.LA_EINVAL                  # no global tokens
    assert _attn(L, d, ext=E(0, ll=FAKE)) == la.LA_EINVAL
    assert _attn(L, d, ext=E(0, sp=16)) == la.LA_EINVAL
    assert _attn(L, d, ext=E(0, sp=-1)) == la.LA_EINVAL
    # globals need a large enough workspace
    assert _attn(L, d, gidx=FAKE, n_global=4) == la.LA_EINVAL
    need = la.la_attn_workspace_size(d, 4)
    assert _attn(L, d, gidx=FAKE, n_global=4,
                 ext=LaAttnExt(0, None, None, None, FAKE, need - 1)) == la.LA_EINVAL
    assert _attn(L, LaDims(1, 65, 128, 64, la.LA_BF16)) == la.LA_EUNSUPPORTED
    # a head of 2^24 rows or more is refused (32-bit byte offsets within a head)
    assert _attn(L, LaDims(1, 1, 1 << 24, 64, la.LA_BF16)) == la.LA_EUNSUPPORTED
    assert "2^24" in la.la_last_error()
    assert _attn(L, LaDims(1, 1, 1 << 24, 64, la.LA_F32)) == la.LA_EUNSUPPORTED
    assert la.la_attn_workspace_size(LaDims(1, 1, 1 << 24, 64, la.LA_BF16), 4) == 0
    # empty tensors are a no-op
    assert _attn(L, LaDims(0, 2, 128, 64, la.LA_BF16), q=None, k=None, v=None, out=None) == la.LA_OK


def test_noalloc_argument_errors(L):
    d = LaDims(1, 2, 128, 64, la.LA_BF16)

    def call(dims=d, gidx=None, n_global=0, ext=None):
        return L.la_attn_forward_noalloc(ctypes.byref(dims), FAKE, FAKE, FAKE, gidx, n_global, 4,
                                         None, 0, None, FAKE, None, None,
                                         ctypes.byref(ext) if ext is not None else None)
    # argument errors as for la_attn_forward
    assert call(dims=LaDims(1, 2, 128, 32, la.LA_BF16)) == la.LA_EUNSUPPORTED
    assert call(n_global=3) == la.LA_EINVAL
    # no workspace may be passed
    assert call(ext=LaAttnExt(0, None, None, None, FAKE, 1024)) == la.LA_EINVAL
    assert "no workspace" in la.la_last_error()
    # a call needing more than the 32 MiB device scratch is refused up front
    big = LaDims(4, 16, 8192, 64, la.LA_BF16)
    assert la.la_attn_workspace_size(big, 1024) > 32 << 20
    assert call(dims=big, gidx=FAKE, n_global=1024) == la.LA_EUNSUPPORTED
    assert "scratch" in la.la_last_error()


def test_dilated_argument_errors(L):
    d = LaDims(1, 2, 256, 64, la.LA_BF16)
    w = (ctypes.c_int32 * 2)(64, 128)
    r = (ctypes.c_int32 * 2)(1, 2)

    def call(dims=d, w=w, r=r, n=2, causal=1, ext=None, q=FAKE):
        return L.la_dilated_forward(ctypes.byref(dims), q, FAKE, FAKE, w, r, n, causal, FAKE, None,
                                    ctypes.byref(ext) if ext is not None else None)
    assert call(dims=LaDims(1, 2, 256, 64, la.LA_F32)) == la.LA_EUNSUPPORTED
    assert call(n=0) == la.LA_EINVAL
    assert call(w=None) == la.LA_EINVAL
    assert call(r=(ctypes.c_int32 * 2)(1, 0)) == la.LA_EINVAL
    big = (ctypes.c_int32 * 17)(*([64] * 17))
    assert call(w=big, r=(ctypes.c_int32 * 17)(*([1] * 17)), n=17) == la.LA_EUNSUPPORTED
    assert call(causal=3) == la.LA_EINVAL
    assert call(q=None) == la.LA_EINVAL
    assert call() == la.LA_EINVAL  # no workspace
    need = la.la_dilated_workspace_size(d, [64, 128], [1, 2])
    assert call(ext=LaDilatedExt(None, FAKE, need - 1)) == la.LA_EINVAL
    assert call(dims=LaDims(1, 1, 1 << 24, 64, la.LA_BF16)) == la.LA_EUNSUPPORTED


def test_fixed_argument_errors(L):
    d = LaDims(1, 2, 1024, 64, la.LA_BF16)
    need = la.la_fixed_workspace_size(d, 256, 64)
    assert need > 0
    ext = LaDilatedExt(None, FAKE, need)

    def call(dims=d, l=256, c=64, causal=1, e=ext):
        return L.la_fixed_forward(ctypes.byref(dims), FAKE, FAKE, FAKE, l, c, causal, FAKE, None,
                                  ctypes.byref(e) if e is not None else None)
    assert call(c=96) == la.LA_EUNSUPPORTED         # summary not a multiple of 64
    assert call(l=300) == la.LA_EUNSUPPORTED        # N not a multiple of the block
    assert call(c=512) == la.LA_EINVAL              # summary longer than the block
    assert call(causal=2) == la.LA_EINVAL
    assert call(e=None) == la.LA_EINVAL             # no workspace
    assert call(dims=LaDims(1, 2, 1024, 64, la.LA_F32)) == la.LA_EUNSUPPORTED
    assert la.la_fixed_workspace_size(d, 256, 96) == 0


def test_backward_argument_errors(L):
    d = LaDims(1, 2, 128, 64, la.LA_BF16)
    need = la.la_attn_backward_workspace_size(d)
    # D_i per row (1 KiB), an int32 rank per position, partial dQ, dK, dV of 128 rows per head,
    # then (bf16) a label table of up to 64 fp32 entries per row
    assert need == 1 * 2 * 128 * 4 + 512 + 3 * 1 * 2 * 128 * 64 * 4 + 1 * 2 * 128 * 64 * 4
    assert la.la_attn_backward_workspace_size(LaDims(1, 2, 128, 64, la.LA_F32)) == 1024 + 512
    assert la.la_attn_backward_workspace_size(LaDims(2, 3, 8192, 64, la.LA_BF16)) == (
        2 * 3 * 8192 * 4 + 8192 * 4 + 3 * 2 * 3 * 2048 * 64 * 4 + 2 * 3 * 8192 * 64 * 4)
    ext = la.LaAttnBwdExt(None, None, None, None, None, None, None, FAKE, need)

    def call(dims=d, q=FAKE, lse=FAKE, dq=FAKE, gidx=None, n_global=0, radius=4, causal=0,
             e=ext):
        return L.la_attn_backward(ctypes.byref(dims) if dims is not None else None, q, FAKE, FAKE,
                                  gidx, n_global, radius, None, causal, FAKE, lse, FAKE, dq, FAKE,
                                  FAKE, None, ctypes.byref(e) if e is not None else None)
    assert call(dims=None) == la.LA_EINVAL
    assert call(q=None) == la.LA_EINVAL
    assert call(lse=None) == la.LA_EINVAL                      # lse is required
    assert call(dq=FAKE + 4) == la.LA_EINVAL                   # misaligned
    assert call(radius=-1) == la.LA_EINVAL
    assert call(causal=2) == la.LA_EINVAL
    assert call(n_global=2) == la.LA_EINVAL                    # count without indices
    assert call(e=None) == la.LA_EINVAL                        # no workspace
    assert call(e=la.LaAttnBwdExt(None, None, None, None, None, None, None, FAKE, need - 1)) \
        == la.LA_EINVAL
    assert call(e=la.LaAttnBwdExt(FAKE, FAKE, FAKE, None, None, None, None, FAKE, need)) \
        == la.LA_EINVAL                                        # qg.. without dqg..
    assert call(e=la.LaAttnBwdExt(None, None, None, None, None, None, FAKE + 2, FAKE, need)) \
        == la.LA_EINVAL                                        # misaligned seg_ids
    # the forward's tables and structured inputs, checked as the forward does
    E = lambda **kw: la.LaAttnBwdExt(None, None, None, None, None, None, None, FAKE, need, **kw)
    assert call(e=E(rel_bias=FAKE)) == la.LA_EINVAL                       # no rel_k
    assert call(e=E(rel_k=2)) == la.LA_EINVAL                             # rel_k, no table
    assert call(e=E(rel_k=2, rel_vec=FAKE + 4)) == la.LA_EINVAL           # misaligned
    assert call(e=E(rel_k=2, rel_bias=FAKE, n_labels=4)) == la.LA_EINVAL  # below 2k+1
    assert call(e=E(rel_k=2, rel_bias=FAKE, n_labels=65)) == la.LA_EUNSUPPORTED
    assert call(e=E(glabel=FAKE)) == la.LA_EINVAL                         # no global tokens
    assert call(e=E(seg_pieces=16)) == la.LA_EINVAL
    assert call(dims=LaDims(1, 2, 128, 32, la.LA_BF16)) == la.LA_EUNSUPPORTED
    assert "D == 64" in la.la_last_error()
    assert call(dims=LaDims(0, 2, 128, 64, la.LA_BF16), e=None) == la.LA_OK  # empty: no-op


def test_dilated_backward_argument_errors(L):
    d = LaDims(1, 2, 256, 64, la.LA_BF16)
    need = la.la_dilated_backward_workspace_size(d)
    assert need == 1 * 2 * 256 * 4                          # D_i per row, 256-byte multiple
    w = (ctypes.c_int32 * 2)(64, 128)
    r = (ctypes.c_int32 * 2)(1, 2)

    def call(dims=d, w=w, r=r, n=2, causal=1, lse=FAKE, ws=FAKE, nbytes=need):
        return L.la_dilated_backward(ctypes.byref(dims), FAKE, FAKE, FAKE, w, r, n, causal, FAKE,
                                     lse, FAKE, FAKE, FAKE, FAKE, None, ws, nbytes)
    assert call(dims=LaDims(1, 2, 256, 64, la.LA_F32)) == la.LA_EUNSUPPORTED
    assert call(n=0) == la.LA_EINVAL
    assert call(r=(ctypes.c_int32 * 2)(1, 0)) == la.LA_EINVAL
    big = (ctypes.c_int32 * 17)(*([64] * 17))
    assert call(w=big, r=(ctypes.c_int32 * 17)(*([1] * 17)), n=17) == la.LA_EUNSUPPORTED
    assert call(causal=2) == la.LA_EINVAL
    assert call(lse=None) == la.LA_EINVAL
    assert call(ws=None) == la.LA_EINVAL
    assert call(nbytes=need - 1) == la.LA_EINVAL
    assert call(dims=LaDims(0, 2, 256, 64, la.LA_BF16), ws=None) == la.LA_OK  # empty: no-op


def test_workspace_sizes(L):
    d = LaDims(2, 12, 4096, 64, la.LA_BF16)
    assert la.la_attn_workspace_size(d, 0) == 0
    # 64 global rows x 8 key chunks of 512 per (b, h): fp32 O plus fp32 lse,
    # then one 64-bit arrival counter word per (b, h) and 128-row tile of
    # global rows, each part padded to 256 bytes
    parts = 2 * 12 * 64 * 8
    assert la.la_attn_workspace_size(d, 64) == parts * 64 * 4 + parts * 4 + 256
    assert la.la_attn_workspace_size(LaDims(1, 1, 10, 64, la.LA_BF16), 11) == 0  # n_global > N
    d5 = LaDims(1, 12, 32768, 64, la.LA_BF16)
    ws = la.la_dilated_workspace_size(d5, [2048, 4096, 8192, 16384, 32768], [1, 2, 4, 6, 12])
    # partial rows of every pattern but the first of dilation 1 (2048, 1), which
    # mixes the others' partials into its own rows instead of writing any
    rows = 12 * (8 * 2048 + 4 * 2048 + 2 * 2731 + 1 * 2731)
    assert ws >= rows * 65 * 4 and ws < rows * 65 * 4 + 1024
