"""sparse_long_sequence_amd — sparse long-sequence attention forward for MI355X (gfx950).

A thin ctypes binding over ``liblongattn.so``, whose C ABI is declared in
``include/longattn.h``. The functions here only marshal arguments: every step
of the attention runs in the library's HIP kernels. PyTorch supplies device
memory and streams. If the library is missing, every call raises
:class:`LaError`; nothing falls back to another implementation.

Entry points (same names as the C ABI):

* :func:`la_attn_forward` — sliding-window (optionally dilated, causal) plus
  global-token attention, with optional separate global projections and a
  per-head scalar relative-position bias (Longformer, ETC).
* :func:`la_dilated_forward` — LongNet's mixture of dilated attentions.
* :func:`la_fixed_forward` — Sparse Transformer's fixed pattern (local block
  plus strided summary positions), LongNet's baseline.
* :func:`la_attn_forward_noalloc` — ``la_attn_forward`` with the library's
  fixed device scratch instead of a workspace (for callers that cannot allocate).
* :func:`la_attn_workspace_size`, :func:`la_dilated_workspace_size`,
  :func:`la_fixed_workspace_size`,
  :func:`la_check_global_idx`, :func:`la_last_error`, :func:`la_version`.

:func:`bind_attn` and :func:`bind_dilated` marshal a call once and return a
:class:`BoundCall` that re-issues it cheaply (the host cost of argument
checking is otherwise comparable to the kernels' own time).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblongattn.so")

LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_EHIP = 0, -1, -2, -3
LA_F32, LA_BF16 = 0, 1


class LaError(RuntimeError):
    """A non-OK status from the library (``status`` holds the code)."""

    def __init__(self, status: int, msg: str):
        super().__init__(f"longattn status {status}: {msg}")
        self.status = status


class LaDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("D", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class LaAttnExt(ctypes.Structure):
    _fields_ = [("rel_k", ctypes.c_int32), ("qg", ctypes.c_void_p), ("kg", ctypes.c_void_p),
                ("vg", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("rel_vec", ctypes.c_void_p),
                ("seg_ids", ctypes.c_void_p), ("glabel", ctypes.c_void_p),
                ("llabel", ctypes.c_void_p), ("n_labels", ctypes.c_int32),
                ("seg_pieces", ctypes.c_int32)]


LABEL_DISTANCE = 0xFE  # a pair keeps its usual clipped-distance label
LABEL_MASKED = 0xFF    # a masked pair (any value >= the vocabulary size but 0xFE)


class LaDilatedExt(ctypes.Structure):
    _fields_ = [("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class LaAttnBwdExt(ctypes.Structure):
    _fields_ = [("qg", ctypes.c_void_p), ("kg", ctypes.c_void_p), ("vg", ctypes.c_void_p),
                ("dqg", ctypes.c_void_p), ("dkg", ctypes.c_void_p), ("dvg", ctypes.c_void_p),
                ("seg_ids", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("rel_k", ctypes.c_int32),
                ("rel_bias", ctypes.c_void_p), ("rel_vec", ctypes.c_void_p),
                ("glabel", ctypes.c_void_p), ("llabel", ctypes.c_void_p),
                ("n_labels", ctypes.c_int32), ("seg_pieces", ctypes.c_int32)]


_i32p = ctypes.POINTER(ctypes.c_int32)
_lib: Optional[ctypes.CDLL] = None

# Every symbol include/longattn.h declares.
EXPORTS = ("la_attn_forward", "la_dilated_forward", "la_fixed_forward", "la_attn_workspace_size",
           "la_dilated_workspace_size", "la_fixed_workspace_size", "la_check_global_idx",
           "la_last_error", "la_version", "la_attn_backward", "la_attn_backward_workspace_size",
           "la_dilated_backward", "la_dilated_backward_workspace_size",
           "la_attn_forward_noalloc")


def lib() -> ctypes.CDLL:
    """Load the HIP library (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LaError(LA_EHIP, f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(or python -m sparse_long_sequence_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    L.la_version.restype = ctypes.c_int32
    L.la_last_error.restype = ctypes.c_char_p
    L.la_attn_forward.restype = ctypes.c_int32
    L.la_attn_forward.argtypes = [ctypes.POINTER(LaDims), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                  _i32p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(LaAttnExt)]
    L.la_attn_forward_noalloc.restype = ctypes.c_int32
    L.la_attn_forward_noalloc.argtypes = L.la_attn_forward.argtypes
    L.la_dilated_forward.restype = ctypes.c_int32
    L.la_dilated_forward.argtypes = [ctypes.POINTER(LaDims), ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(LaDilatedExt)]
    L.la_fixed_forward.restype = ctypes.c_int32
    L.la_fixed_forward.argtypes = [ctypes.POINTER(LaDims), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(LaDilatedExt)]
    L.la_fixed_workspace_size.restype = ctypes.c_size_t
    L.la_fixed_workspace_size.argtypes = [ctypes.POINTER(LaDims), ctypes.c_int32, ctypes.c_int32]
    L.la_attn_workspace_size.restype = ctypes.c_size_t
    L.la_attn_workspace_size.argtypes = [ctypes.POINTER(LaDims), ctypes.c_int32, ctypes.c_int32]
    L.la_dilated_workspace_size.restype = ctypes.c_size_t
    L.la_dilated_workspace_size.argtypes = [ctypes.POINTER(LaDims), _i32p, _i32p, ctypes.c_int32]
    L.la_attn_backward.restype = ctypes.c_int32
    L.la_attn_backward.argtypes = [ctypes.POINTER(LaDims), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   _i32p, ctypes.c_int32] + [ctypes.c_void_p] * 6 + [
                                   ctypes.c_void_p, ctypes.POINTER(LaAttnBwdExt)]
    L.la_attn_backward_workspace_size.restype = ctypes.c_size_t
    L.la_attn_backward_workspace_size.argtypes = [ctypes.POINTER(LaDims)]
    L.la_dilated_backward.restype = ctypes.c_int32
    L.la_dilated_backward.argtypes = [ctypes.POINTER(LaDims), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, _i32p, _i32p, ctypes.c_int32,
                                      ctypes.c_int32] + [ctypes.c_void_p] * 6 + [
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]
    L.la_dilated_backward_workspace_size.restype = ctypes.c_size_t
    L.la_dilated_backward_workspace_size.argtypes = [ctypes.POINTER(LaDims)]
    L.la_check_global_idx.restype = ctypes.c_int32
    L.la_check_global_idx.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p]
    _lib = L
    return L


def la_version() -> int:
    return int(lib().la_version())


def la_last_error() -> str:
    return lib().la_last_error().decode()


def _check(status: int):
    if status != LA_OK:
        raise LaError(status, la_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise LaError(LA_EINVAL, f"unsupported dtype {t.dtype}")


def _dims(q: torch.Tensor) -> LaDims:
    if q.dim() != 4:
        raise LaError(LA_EINVAL, "tensors must be [B, H, N, D]")
    B, H, N, D = q.shape
    return LaDims(B, H, N, D, _dtype_code(q))


def _dev(t: Optional[torch.Tensor], like: torch.Tensor, name: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda or not t.is_contiguous() or t.shape != like.shape or t.dtype != like.dtype:
        raise LaError(LA_EINVAL, f"{name} must be a contiguous device tensor shaped and typed like q")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _host_i32(vals: Sequence[int]):
    arr = (ctypes.c_int32 * len(vals))(*[int(x) for x in vals])
    return arr


def la_attn_workspace_size(dims: LaDims, n_global: int, has_separate_global: bool = False) -> int:
    return int(lib().la_attn_workspace_size(ctypes.byref(dims), int(n_global),
                                            int(bool(has_separate_global))))


def la_dilated_workspace_size(dims: LaDims, seg_lens: Sequence[int], dil_rates: Sequence[int]) -> int:
    return int(lib().la_dilated_workspace_size(ctypes.byref(dims), _host_i32(seg_lens),
                                               _host_i32(dil_rates), len(seg_lens)))


def _workspace(nbytes: int, device, given: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    if given is not None:
        if given.numel() * given.element_size() < nbytes or not given.is_cuda:
            raise LaError(LA_EINVAL, "workspace tensor too small")
        return given
    # torch's caching allocator returns 512-byte aligned blocks; the library
    # needs no particular contents in a workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


class BoundCall:
    """One forward call with its arguments already marshalled.

    Built by :func:`bind_attn` / :func:`bind_dilated`; calling it re-issues the
    same C call (same tensors, workspace and stream) with no Python-side
    checks, for loops that repeat one call. The tensors it refers to are kept
    alive by the object.
    """

    def __init__(self, fn, args, keep, out, lse):
        self._fn, self._args, self._keep = fn, args, keep
        self.out, self.lse = out, lse

    def __call__(self) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
        st = self._fn(*self._args)
        if st != LA_OK:
            _check(st)
        return self.out, self.lse


class BoundBackward(BoundCall):
    """A marshalled :func:`la_attn_backward` call; calling it re-issues the call
    and returns its gradient tensors (``grads``), which every call overwrites."""

    def __init__(self, fn, args, keep, grads):
        super().__init__(fn, args, keep, None, None)
        self.grads = grads

    def __call__(self) -> Tuple[torch.Tensor, ...]:
        super().__call__()
        return self.grads


class _Labels:
    """Checked bias tables and label matrices of one call (contiguous tensors
    and what the C structs take)."""

    def __init__(self, rb, rv, rk, n_labels, gl, ll):
        self.rb, self.rv, self.rk, self.n_labels, self.gl, self.ll = rb, rv, rk, n_labels, gl, ll

    @staticmethod
    def ptr(t):
        return None if t is None else t.data_ptr()


def _labels(dims: LaDims, n_global: int, rel_bias, rel_vec, rel_k, glabel, llabel) -> _Labels:
    V = None
    if rel_bias is not None:
        if rel_bias.dtype != torch.float32 or not rel_bias.is_cuda or rel_bias.dim() != 2 \
                or rel_bias.shape[0] != dims.H:
            raise LaError(LA_EINVAL, "rel_bias must be a device fp32 [H, V] tensor")
        V = rel_bias.shape[1]
        rel_bias = rel_bias.contiguous()
    if rel_vec is not None:
        if rel_vec.dtype != torch.float32 or not rel_vec.is_cuda or rel_vec.dim() != 3 \
                or rel_vec.shape[0] != dims.H or rel_vec.shape[2] != dims.D:
            raise LaError(LA_EINVAL, "rel_vec must be a device fp32 [H, V, D] tensor")
        if V is not None and rel_vec.shape[1] != V:
            raise LaError(LA_EINVAL, "rel_bias and rel_vec need the same vocabulary")
        V = rel_vec.shape[1]
        rel_vec = rel_vec.contiguous()
    rk, n_labels = 0, 0
    if V is not None:
        if rel_k is None:
            if V % 2 != 1:
                raise LaError(LA_EINVAL, "give rel_k with a vocabulary of structural labels")
            rel_k = (V - 1) // 2
        rk = int(rel_k)
        n_labels = 0 if V == 2 * rk + 1 else V
    mats = []
    for name, t, shape in (("glabel", glabel, (dims.B, n_global, dims.N)),
                           ("llabel", llabel, (dims.B, dims.N, n_global))):
        if t is not None:
            if t.dtype != torch.uint8 or not t.is_cuda or tuple(t.shape) != shape:
                raise LaError(LA_EINVAL, f"{name} must be a device uint8 {list(shape)} tensor")
            t = t.contiguous()
        mats.append(t)
    return _Labels(rel_bias, rel_vec, rk, n_labels, mats[0], mats[1])


def bind_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
              global_idx: Optional[torch.Tensor] = None, radius: int = 0,
              dilation: Optional[Sequence[int]] = None, causal: bool = False,
              rel_bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None, qg: Optional[torch.Tensor] = None,
              kg: Optional[torch.Tensor] = None, vg: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None,
              want_lse: bool = True, rel_vec: Optional[torch.Tensor] = None,
              seg_ids: Optional[torch.Tensor] = None, noalloc: bool = False,
              rel_k: Optional[int] = None, glabel: Optional[torch.Tensor] = None,
              llabel: Optional[torch.Tensor] = None, seg_pieces: int = 0) -> BoundCall:
    """Validate and marshal a :func:`la_attn_forward` call without issuing it.

    With structural labels the tables are ``rel_bias [H, V]`` and ``rel_vec
    [H, V, D]`` for a vocabulary of V labels (the 2k+1 distance labels, then
    the structural ones; give ``rel_k`` when V > 2k+1). ``glabel`` (device
    uint8 ``[B, n_global, N]``) and ``llabel`` (``[B, N, n_global]``) give per-pair
    labels of the pieces with a global token; ``seg_pieces`` selects the pieces
    ``seg_ids`` masks (bits g2g 1, g2l 2, l2g 4, l2l 8; 0 = all).

    ``noalloc`` marshals :func:`la_attn_forward_noalloc` instead (no workspace:
    the library's fixed device scratch).

    ``rel_vec`` is a device fp32 ``[H, 2k+1, D]`` tensor of key-side label
    vectors (with or without ``rel_bias``, same k). ``seg_ids`` is a device
    int32 ``[B, N]`` tensor of segment ids: pairs across segments are masked."""
    dims = _dims(q)
    for name, t in (("k", k), ("v", v)):
        _dev(t, q, name)
    qptr = _dev(q, q, "q")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, q, "out")
    if want_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != tuple(q.shape[:3])):
        raise LaError(LA_EINVAL, "lse must be a contiguous fp32 [B, H, N] tensor")
    n_global = 0
    gptr = 0
    if global_idx is not None:
        if global_idx.dtype != torch.int32 or not global_idx.is_cuda or global_idx.dim() != 1:
            raise LaError(LA_EINVAL, "global_idx must be a 1-D device int32 tensor")
        n_global = global_idx.numel()
        gptr = global_idx.data_ptr() if n_global else 0
    dil = None if dilation is None else _host_i32(dilation)
    if dilation is not None and len(dilation) != dims.H:
        raise LaError(LA_EINVAL, "dilation needs one entry per head")
    lab = _labels(dims, n_global, rel_bias, rel_vec, rel_k, glabel, llabel)
    sptr = 0
    if seg_ids is not None:
        if seg_ids.dtype != torch.int32 or not seg_ids.is_cuda \
                or tuple(seg_ids.shape) != (dims.B, dims.N):
            raise LaError(LA_EINVAL, "seg_ids must be a device int32 [B, N] tensor")
        seg_ids = seg_ids.contiguous()
        sptr = seg_ids.data_ptr()
    sep = qg is not None
    if noalloc:
        if workspace is not None:
            raise LaError(LA_EINVAL, "la_attn_forward_noalloc takes no workspace")
        ws = None
    else:
        ws = _workspace(la_attn_workspace_size(dims, n_global, sep), q.device, workspace)
    ext = LaAttnExt(lab.rk, _dev(qg, q, "qg") or None, _dev(kg, q, "kg") or None,
                    _dev(vg, q, "vg") or None, ws.data_ptr() if ws is not None else None,
                    ws.numel() if ws is not None else 0, lab.ptr(lab.rv), sptr or None,
                    lab.ptr(lab.gl), lab.ptr(lab.ll), lab.n_labels, int(seg_pieces))
    args = (ctypes.byref(dims), qptr, k.data_ptr(), v.data_ptr(), gptr or None, n_global,
            int(radius), dil, int(bool(causal)), lab.ptr(lab.rb), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, _stream(q, stream), ctypes.byref(ext))
    keep = (dims, ext, dil, q, k, v, global_idx, lab, seg_ids, qg, kg, vg, ws)
    fn = lib().la_attn_forward_noalloc if noalloc else lib().la_attn_forward
    return BoundCall(fn, args, keep, out, lse)


def la_attn_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                    global_idx: Optional[torch.Tensor] = None, radius: int = 0,
                    dilation: Optional[Sequence[int]] = None, causal: bool = False,
                    rel_bias: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, qg: Optional[torch.Tensor] = None,
                    kg: Optional[torch.Tensor] = None, vg: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    want_lse: bool = True, rel_vec: Optional[torch.Tensor] = None,
                    seg_ids: Optional[torch.Tensor] = None, rel_k: Optional[int] = None,
                    glabel: Optional[torch.Tensor] = None, llabel: Optional[torch.Tensor] = None,
                    seg_pieces: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Band + global attention; returns ``(out, lse)``.

    ``global_idx`` is a device int32 tensor of strictly increasing positions.
    ``rel_bias`` is a device fp32 ``[H, 2k+1]`` table and ``rel_vec`` a device
    fp32 ``[H, 2k+1, D]`` table of key-side label vectors. ``seg_ids`` (device
    int32 ``[B, N]``) masks pairs across segments. ``out``, ``lse`` and
    the workspace are allocated with torch when not given. Structural labels
    and piece-selected segment masks: see :func:`bind_attn`.
    """
    return bind_attn(q, k, v, global_idx, radius, dilation, causal, rel_bias, out, lse, qg, kg,
                     vg, workspace, stream, want_lse, rel_vec, seg_ids, False, rel_k, glabel,
                     llabel, seg_pieces)()


def la_attn_forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            global_idx: Optional[torch.Tensor] = None, radius: int = 0,
                            dilation: Optional[Sequence[int]] = None, causal: bool = False,
                            rel_bias: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            qg: Optional[torch.Tensor] = None, kg: Optional[torch.Tensor] = None,
                            vg: Optional[torch.Tensor] = None, stream=None, want_lse: bool = True,
                            rel_vec: Optional[torch.Tensor] = None,
                            seg_ids: Optional[torch.Tensor] = None
                            ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """:func:`la_attn_forward` without a workspace: the library's fixed device
    scratch (32 MiB per GPU) holds the global rows' partials. The C call
    allocates nothing; ``out`` and ``lse`` are still allocated here when not
    given. Calls that overlap in time on one GPU race."""
    return bind_attn(q, k, v, global_idx, radius, dilation, causal, rel_bias, out, lse, qg, kg,
                     vg, None, stream, want_lse, rel_vec, seg_ids, noalloc=True)()


def bind_dilated(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 seg_lens: Sequence[int], dil_rates: Sequence[int], causal: bool = True,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None,
                 want_lse: bool = True) -> BoundCall:
    """Validate and marshal a :func:`la_dilated_forward` call without issuing it."""
    dims = _dims(q)
    for name, t in (("k", k), ("v", v)):
        _dev(t, q, name)
    qptr = _dev(q, q, "q")
    if len(seg_lens) != len(dil_rates):
        raise LaError(LA_EINVAL, "seg_lens and dil_rates differ in length")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, q, "out")
    if want_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    nbytes = la_dilated_workspace_size(dims, seg_lens, dil_rates) if len(seg_lens) else 0
    ws = _workspace(nbytes, q.device, workspace)
    ext = LaDilatedExt(lse.data_ptr() if lse is not None else None,
                       ws.data_ptr() if ws is not None else None,
                       ws.numel() if ws is not None else 0)
    w_arr, r_arr = _host_i32(seg_lens), _host_i32(dil_rates)
    args = (ctypes.byref(dims), qptr, k.data_ptr(), v.data_ptr(), w_arr, r_arr, len(seg_lens),
            int(bool(causal)), out.data_ptr(), _stream(q, stream), ctypes.byref(ext))
    keep = (dims, ext, w_arr, r_arr, q, k, v, ws)
    return BoundCall(lib().la_dilated_forward, args, keep, out, lse)


def la_dilated_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       seg_lens: Sequence[int], dil_rates: Sequence[int], causal: bool = True,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None,
                       want_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """LongNet dilated attention mixture; returns ``(out, lse)``."""
    return bind_dilated(q, k, v, seg_lens, dil_rates, causal, out, lse, workspace, stream,
                        want_lse)()


def la_fixed_workspace_size(dims: LaDims, block_len: int, summary_len: int) -> int:
    return int(lib().la_fixed_workspace_size(ctypes.byref(dims), int(block_len), int(summary_len)))


def bind_fixed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_len: int,
               summary_len: int, causal: bool = True, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None, want_lse: bool = True) -> BoundCall:
    """Validate and marshal a :func:`la_fixed_forward` call without issuing it."""
    dims = _dims(q)
    for name, t in (("k", k), ("v", v)):
        _dev(t, q, name)
    qptr = _dev(q, q, "q")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, q, "out")
    if want_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    ws = _workspace(la_fixed_workspace_size(dims, block_len, summary_len), q.device, workspace)
    ext = LaDilatedExt(lse.data_ptr() if lse is not None else None,
                       ws.data_ptr() if ws is not None else None,
                       ws.numel() if ws is not None else 0)
    args = (ctypes.byref(dims), qptr, k.data_ptr(), v.data_ptr(), int(block_len),
            int(summary_len), int(bool(causal)), out.data_ptr(), _stream(q, stream),
            ctypes.byref(ext))
    keep = (dims, ext, q, k, v, ws)
    return BoundCall(lib().la_fixed_forward, args, keep, out, lse)


def la_fixed_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_len: int,
                     summary_len: int, causal: bool = True, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None, want_lse: bool = True
                     ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Sparse Transformer fixed pattern (local block plus strided summary
    positions); returns ``(out, lse)``."""
    return bind_fixed(q, k, v, block_len, summary_len, causal, out, lse, workspace, stream,
                      want_lse)()


def la_attn_backward_workspace_size(dims: LaDims) -> int:
    return int(lib().la_attn_backward_workspace_size(ctypes.byref(dims)))


def bind_attn_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor, dout: torch.Tensor,
                       global_idx: Optional[torch.Tensor] = None, radius: int = 0,
                       dilation: Optional[Sequence[int]] = None, causal: bool = False,
                       qg: Optional[torch.Tensor] = None, kg: Optional[torch.Tensor] = None,
                       vg: Optional[torch.Tensor] = None, seg_ids: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None,
                       rel_bias: Optional[torch.Tensor] = None,
                       rel_vec: Optional[torch.Tensor] = None, rel_k: Optional[int] = None,
                       glabel: Optional[torch.Tensor] = None,
                       llabel: Optional[torch.Tensor] = None,
                       seg_pieces: int = 0) -> BoundBackward:
    """Validate and marshal a :func:`la_attn_backward` call without issuing it.

    ``out`` and ``lse`` are the forward's outputs for the same arguments and
    ``dout`` the loss gradient w.r.t. ``out`` (dtype of ``q``). The call's
    results are fp32 ``(dq, dk, dv)``, plus ``(dqg, dkg, dvg)`` with separate
    global projections. The bias tables, label matrices and segment pieces are
    those given to the forward (see :func:`bind_attn`); the tables are not
    differentiated."""
    dims = _dims(q)
    ptrs = [_dev(t, q, name) for name, t in (("q", q), ("k", k), ("v", v), ("out", out),
                                             ("dout", dout))]
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() \
            or tuple(lse.shape) != tuple(q.shape[:3]):
        raise LaError(LA_EINVAL, "lse must be a contiguous device fp32 [B, H, N] tensor")
    n_global, gptr = 0, 0
    if global_idx is not None:
        if global_idx.dtype != torch.int32 or not global_idx.is_cuda or global_idx.dim() != 1:
            raise LaError(LA_EINVAL, "global_idx must be a 1-D device int32 tensor")
        n_global = global_idx.numel()
        gptr = global_idx.data_ptr() if n_global else 0
    if dilation is not None and len(dilation) != dims.H:
        raise LaError(LA_EINVAL, "dilation needs one entry per head")
    dil = None if dilation is None else _host_i32(dilation)
    lab = _labels(dims, n_global, rel_bias, rel_vec, rel_k, glabel, llabel)
    sptr = 0
    if seg_ids is not None:
        if seg_ids.dtype != torch.int32 or not seg_ids.is_cuda \
                or tuple(seg_ids.shape) != (dims.B, dims.N):
            raise LaError(LA_EINVAL, "seg_ids must be a device int32 [B, N] tensor")
        seg_ids = seg_ids.contiguous()
        sptr = seg_ids.data_ptr()
    sep = qg is not None
    grads = [torch.empty(q.shape, dtype=torch.float32, device=q.device)
             for _ in range(6 if sep else 3)]
    gp = [None] * 6
    if sep:
        gp = [_dev(qg, q, "qg"), _dev(kg, q, "kg"), _dev(vg, q, "vg")] + \
             [t.data_ptr() for t in grads[3:]]
    ws = _workspace(la_attn_backward_workspace_size(dims), q.device, workspace)
    ext = LaAttnBwdExt(*gp, sptr or None, ws.data_ptr() if ws is not None else None,
                       ws.numel() if ws is not None else 0, lab.rk, lab.ptr(lab.rb),
                       lab.ptr(lab.rv), lab.ptr(lab.gl), lab.ptr(lab.ll), lab.n_labels,
                       int(seg_pieces))
    args = (ctypes.byref(dims), ptrs[0], ptrs[1], ptrs[2], gptr or None, n_global, int(radius),
            dil, int(bool(causal)), ptrs[3], lse.data_ptr(), ptrs[4],
            grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), _stream(q, stream),
            ctypes.byref(ext))
    keep = (dims, ext, dil, q, k, v, out, lse, dout, global_idx, seg_ids, qg, kg, vg, ws, lab)
    return BoundBackward(lib().la_attn_backward, args, keep, tuple(grads))


def la_attn_backward(q, k, v, out, lse, dout, global_idx=None, radius: int = 0, dilation=None,
                     causal: bool = False, qg=None, kg=None, vg=None, seg_ids=None,
                     workspace=None, stream=None, rel_bias=None, rel_vec=None, rel_k=None,
                     glabel=None, llabel=None, seg_pieces: int = 0):
    """One backward call; returns fp32 ``(dq, dk, dv)`` or, with separate global
    projections, ``(dq, dk, dv, dqg, dkg, dvg)``."""
    return bind_attn_backward(q, k, v, out, lse, dout, global_idx, radius, dilation, causal,
                              qg, kg, vg, seg_ids, workspace, stream, rel_bias, rel_vec, rel_k,
                              glabel, llabel, seg_pieces)()


def la_dilated_backward_workspace_size(dims: LaDims) -> int:
    return int(lib().la_dilated_backward_workspace_size(ctypes.byref(dims)))


def bind_dilated_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                          lse: torch.Tensor, dout: torch.Tensor, seg_lens: Sequence[int],
                          dil_rates: Sequence[int], causal: bool = True,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> BoundBackward:
    """Validate and marshal a :func:`la_dilated_backward` call; calling the
    result returns fp32 ``(dq, dk, dv)``. ``out`` and ``lse`` are the forward's."""
    dims = _dims(q)
    ptrs = [_dev(t, q, name) for name, t in (("q", q), ("k", k), ("v", v), ("out", out),
                                             ("dout", dout))]
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous() \
            or tuple(lse.shape) != tuple(q.shape[:3]):
        raise LaError(LA_EINVAL, "lse must be a contiguous device fp32 [B, H, N] tensor")
    if len(seg_lens) != len(dil_rates):
        raise LaError(LA_EINVAL, "seg_lens and dil_rates differ in length")
    w, r = _host_i32(seg_lens), _host_i32(dil_rates)
    grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(3))
    ws = _workspace(la_dilated_backward_workspace_size(dims), q.device, workspace)
    args = (ctypes.byref(dims), ptrs[0], ptrs[1], ptrs[2], w, r, len(seg_lens), int(bool(causal)),
            ptrs[3], lse.data_ptr(), ptrs[4], grads[0].data_ptr(), grads[1].data_ptr(),
            grads[2].data_ptr(), _stream(q, stream), ws.data_ptr() if ws is not None else None,
            ws.numel() if ws is not None else 0)
    keep = (dims, w, r, q, k, v, out, lse, dout, ws)
    return BoundBackward(lib().la_dilated_backward, args, keep, grads)


def la_dilated_backward(q, k, v, out, lse, dout, seg_lens, dil_rates, causal: bool = True,
                        workspace=None, stream=None):
    """One LongNet backward call; returns fp32 ``(dq, dk, dv)``."""
    return bind_dilated_backward(q, k, v, out, lse, dout, seg_lens, dil_rates, causal, workspace,
                                 stream)()


def la_check_global_idx(global_idx: torch.Tensor, N: int, stream=None) -> bool:
    """Synchronous check that ``global_idx`` is strictly increasing in [0, N)."""
    n = global_idx.numel()
    st = lib().la_check_global_idx(global_idx.data_ptr() if n else None, n, int(N),
                                   _stream(global_idx, stream))
    if st == LA_EINVAL:
        return False
    _check(st)
    return True
