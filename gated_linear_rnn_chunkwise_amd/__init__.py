"""Chunkwise gated linear attention forward pass for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libgla.so`` (declared in ``include/gla.h``):
this module only marshals arguments (device pointers, sizes, the current HIP stream);
every step of the computation runs in the library's HIP kernels.  PyTorch supplies device
memory and streams.  If the built library is missing, :func:`load` raises: there is no
fallback implementation.

    import gated_linear_rnn_chunkwise_amd as gla
    out, final_state = gla.fwd(q, k, v, log_alpha, chunk=64)

Gate kinds follow the shape of ``log_alpha``: ``None`` (ungated), ``[B,H,L,Dk]``
(per channel), ``[B,H,L]`` (per head and token) or ``[H]`` (fixed per head).
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgla.so")

GLA_OK, GLA_ERR_INVALID_ARG, GLA_ERR_UNSUPPORTED, GLA_ERR_WORKSPACE, GLA_ERR_HIP = 0, -1, -2, -3, -4
DTYPE_BF16, DTYPE_F32 = 0, 1
GATE_NONE, GATE_CHANNEL, GATE_HEAD, GATE_HEAD_CONST = 0, 1, 2, 3
FLAG_TILE_PAIRS = 1
FLAG_QUERY_TILES = 2
GATE_NAMES = {"none": GATE_NONE, "channel": GATE_CHANNEL, "head": GATE_HEAD, "head_const": GATE_HEAD_CONST}

# Entry points declared in include/gla.h.
EXPORTS = ("gla_fwd", "gla_fwd_ex", "gla_fwd_noalloc", "gla_workspace_size", "gla_query_plan", "gla_step",
           "gla_bwd", "gla_bwd_workspace_size", "gla_delta_fwd", "gla_mlstm_fwd", "gla_status_string",
           "gla_version")
NOALLOC_SCRATCH_BYTES = 32 << 20  # GLA_NOALLOC_SCRATCH_BYTES


class GlaDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32), ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("gate_kind", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("log_alpha", ctypes.c_void_p), ("log_ig", ctypes.c_void_p), ("initial_state", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("seg_chunks", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class GlaPlan(ctypes.Structure):
    _fields_ = [
        ("seg_chunks", ctypes.c_int32), ("n_seg", ctypes.c_int32), ("dv_tiles", ctypes.c_int32),
        ("tiles_per_chunk", ctypes.c_int32), ("grid_state", ctypes.c_int32), ("grid_scan", ctypes.c_int32),
        ("grid_out", ctypes.c_int32), ("tile_pairs", ctypes.c_int32), ("query_tiles", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class GlaStepDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("gate_kind", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("log_alpha", ctypes.c_void_p), ("log_ig", ctypes.c_void_p),
        ("state", ctypes.c_void_p), ("out", ctypes.c_void_p),
    ]


class GlaBwdDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("gate_kind", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("log_alpha", ctypes.c_void_p), ("log_ig", ctypes.c_void_p), ("initial_state", ctypes.c_void_p),
        ("dout", ctypes.c_void_p), ("dfinal_state", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dlog_alpha", ctypes.c_void_p), ("dlog_ig", ctypes.c_void_p), ("dinitial_state", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class GlaDeltaDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32), ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("gate_kind", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("log_alpha", ctypes.c_void_p), ("initial_state", ctypes.c_void_p),
        ("out", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
    ]


class GlaMlstmDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32), ("Dk", ctypes.c_int32),
        ("Dv", ctypes.c_int32), ("chunk", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("log_f", ctypes.c_void_p),
        ("log_i", ctypes.c_void_p), ("initial_C", ctypes.c_void_p), ("initial_n", ctypes.c_void_p),
        ("initial_m", ctypes.c_void_p), ("out", ctypes.c_void_p), ("final_C", ctypes.c_void_p),
        ("final_n", ctypes.c_void_p), ("final_m", ctypes.c_void_p),
    ]


class GlaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (status %d)" % (what or "gla", status_string(status), status))


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH):
    """Load ``libgla.so`` (built by ``gated_linear_rnn_chunkwise_amd.build``); raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libgla.so not built: run `python -m gated_linear_rnn_chunkwise_amd.build` "
                               "(expected at %s)" % path)
        lib = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.gla_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.gla_fwd.restype = i32
        lib.gla_fwd_ex.argtypes = [ctypes.POINTER(GlaDesc), vp]
        lib.gla_fwd_ex.restype = i32
        lib.gla_fwd_noalloc.argtypes = [ctypes.POINTER(GlaDesc), vp]
        lib.gla_fwd_noalloc.restype = i32
        lib.gla_workspace_size.argtypes = [ctypes.POINTER(GlaDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.gla_workspace_size.restype = i32
        lib.gla_query_plan.argtypes = [ctypes.POINTER(GlaDesc), ctypes.POINTER(GlaPlan)]
        lib.gla_query_plan.restype = i32
        lib.gla_step.argtypes = [ctypes.POINTER(GlaStepDesc), vp]
        lib.gla_step.restype = i32
        lib.gla_bwd.argtypes = [ctypes.POINTER(GlaBwdDesc), vp]
        lib.gla_bwd.restype = i32
        lib.gla_bwd_workspace_size.argtypes = [ctypes.POINTER(GlaBwdDesc), ctypes.POINTER(ctypes.c_size_t)]
        lib.gla_bwd_workspace_size.restype = i32
        lib.gla_delta_fwd.argtypes = [ctypes.POINTER(GlaDeltaDesc), vp]
        lib.gla_delta_fwd.restype = i32
        lib.gla_mlstm_fwd.argtypes = [ctypes.POINTER(GlaMlstmDesc), vp]
        lib.gla_mlstm_fwd.restype = i32
        lib.gla_status_string.argtypes = [i32]
        lib.gla_status_string.restype = ctypes.c_char_p
        lib.gla_version.argtypes = []
        lib.gla_version.restype = i32
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().gla_status_string(int(status)).decode()


def version() -> int:
    return int(load().gla_version())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return int(t.data_ptr())


def gate_kind_of(log_alpha, B: int, H: int, L: int, Dk: int) -> int:
    if log_alpha is None:
        return GATE_NONE
    shape = tuple(log_alpha.shape)
    if shape == (B, H, L, Dk):
        return GATE_CHANNEL
    if shape == (B, H, L):
        return GATE_HEAD
    if shape == (H,):
        return GATE_HEAD_CONST
    raise ValueError("log_alpha shape %s matches no gate layout for B=%d H=%d L=%d Dk=%d" % (shape, B, H, L, Dk))


def make_desc(q, k, v, log_alpha=None, log_ig=None, initial_state=None, out=None, final_state=None, chunk=64,
              seg_chunks=0, workspace=None, workspace_bytes=0, gate_kind=None, tile_pairs=False,
              query_tiles=False) -> GlaDesc:
    """Fill a :class:`GlaDesc` from tensors (shapes read from q and v)."""
    import torch

    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    d = GlaDesc()
    d.B, d.H, d.L, d.Dk, d.Dv, d.chunk = B, H, L, Dk, Dv, int(chunk)
    if q.dtype == torch.bfloat16:
        d.in_dtype = DTYPE_BF16
    elif q.dtype == torch.float32:
        d.in_dtype = DTYPE_F32
    else:
        raise TypeError("q, k, v must be bf16 or fp32, got %s" % q.dtype)
    d.gate_kind = gate_kind_of(log_alpha, B, H, L, Dk) if gate_kind is None else int(gate_kind)
    d.q, d.k, d.v = _ptr(q), _ptr(k), _ptr(v)
    d.log_alpha, d.log_ig, d.initial_state = _ptr(log_alpha), _ptr(log_ig), _ptr(initial_state)
    d.out, d.final_state = _ptr(out), _ptr(final_state)
    d.seg_chunks = int(seg_chunks)
    d.flags = (FLAG_TILE_PAIRS if tile_pairs else 0) | (FLAG_QUERY_TILES if query_tiles else 0)
    d.workspace = _ptr(workspace)
    d.workspace_bytes = int(workspace_bytes)
    return d


def _check_shape(t, shape, name):
    """Raise ValueError unless tensor ``t`` (or None) has exactly ``shape``."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _check_fwd_shapes(q, k, v, log_alpha, log_ig, initial_state, out, fin):
    """Every tensor of a forward call against the sizes taken from q and v.  The kernels size
    their memory ranges from these sizes, so a shorter tensor would be read or written past
    its end."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, H, L, D]")
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    _check_shape(k, (B, H, L, Dk), "k")
    _check_shape(v, (B, H, L, Dv), "v")
    if log_alpha is not None:
        gate_kind_of(log_alpha, B, H, L, Dk)  # raises when no gate layout matches
    _check_shape(log_ig, (B, H, L), "log_ig")
    _check_shape(initial_state, (B, H, Dk, Dv), "initial_state")
    _check_shape(out, (B, H, L, Dv), "out")
    _check_shape(fin, (B, H, Dk, Dv), "final_state")


def _check_tensors(q, k, v, *others):
    import torch

    for t in (q, k, v) + tuple(o for o in others if o is not None):
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    for t in others:
        if t is not None and t.dtype != torch.float32:
            raise TypeError("gates, states and outputs are fp32")


def fwd(q, k, v, log_alpha=None, *, log_ig=None, initial_state=None, chunk: int = 64, final_state: bool = True,
        seg_chunks: int = 0, out=None, workspace=None, stream=None, tile_pairs: bool = False,
        query_tiles: bool = False):
    """Gated linear attention forward on the current HIP stream.

    ``tile_pairs`` selects the tiled large-chunk form for chunks of more than 64 tokens
    (``GLA_FLAG_TILE_PAIRS``); ``query_tiles`` the same form with one workgroup per query
    tile against materialised chunk-start states (``GLA_FLAG_QUERY_TILES``).  Returns ``(out [B,H,L,Dv] fp32, final_state [B,H,Dk,Dv] fp32 or None)``."""
    import torch

    lib = load()
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    _check_fwd_shapes(q, k, v, log_alpha, log_ig, initial_state, out, None)
    if out is None:
        out = torch.empty((B, H, L, Dv), dtype=torch.float32, device=q.device)
    fin = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device) if final_state else None
    _check_tensors(q, k, v, log_alpha, log_ig, initial_state, out, fin)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = make_desc(q, k, v, log_alpha, log_ig, initial_state, out, fin, chunk, seg_chunks, workspace, ws_bytes,
                  tile_pairs=tile_pairs, query_tiles=query_tiles)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib.gla_fwd_ex(ctypes.byref(d), ctypes.c_void_p(s.cuda_stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_fwd_ex")
    return out, fin


def fwd_noalloc(q, k, v, log_alpha=None, *, log_ig=None, initial_state=None, chunk: int = 64, out=None,
                final_state=None, seg_chunks: int = 0, stream=None, tile_pairs: bool = False,
                query_tiles: bool = False):
    """The forward pass through ``gla_fwd_noalloc``: no device memory is allocated by the
    library (its scratch is a fixed per-GPU array).  ``out`` and ``final_state`` (or None)
    are caller tensors, so nothing at all is allocated when both are given.  Returns
    ``(out, final_state)``."""
    import torch

    lib = load()
    _check_fwd_shapes(q, k, v, log_alpha, log_ig, initial_state, out, final_state)
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    if out is None:
        out = torch.empty((B, H, L, Dv), dtype=torch.float32, device=q.device)
    _check_tensors(q, k, v, log_alpha, log_ig, initial_state, out, final_state)
    d = make_desc(q, k, v, log_alpha, log_ig, initial_state, out, final_state, chunk, seg_chunks, None, 0,
                  tile_pairs=tile_pairs, query_tiles=query_tiles)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib.gla_fwd_noalloc(ctypes.byref(d), ctypes.c_void_p(s.cuda_stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_fwd_noalloc")
    return out, final_state


def make_bwd_desc(q, k, v, dout, dq, dk, dv, log_alpha=None, log_ig=None, initial_state=None, dfinal_state=None,
                  dlog_alpha=None, dlog_ig=None, dinitial_state=None, workspace=None, workspace_bytes=0,
                  gate_kind=None) -> GlaBwdDesc:
    """Fill a :class:`GlaBwdDesc` from tensors (shapes read from q and v)."""
    import torch

    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    d = GlaBwdDesc()
    d.B, d.H, d.L, d.Dk, d.Dv = B, H, L, Dk, Dv
    if q.dtype == torch.bfloat16:
        d.in_dtype = DTYPE_BF16
    elif q.dtype == torch.float32:
        d.in_dtype = DTYPE_F32
    else:
        raise TypeError("q, k, v must be bf16 or fp32, got %s" % q.dtype)
    d.gate_kind = gate_kind_of(log_alpha, B, H, L, Dk) if gate_kind is None else int(gate_kind)
    d.q, d.k, d.v = _ptr(q), _ptr(k), _ptr(v)
    d.log_alpha, d.log_ig, d.initial_state = _ptr(log_alpha), _ptr(log_ig), _ptr(initial_state)
    d.dout, d.dfinal_state = _ptr(dout), _ptr(dfinal_state)
    d.dq, d.dk, d.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    d.dlog_alpha, d.dlog_ig, d.dinitial_state = _ptr(dlog_alpha), _ptr(dlog_ig), _ptr(dinitial_state)
    d.workspace = _ptr(workspace) if workspace is not None else None
    d.workspace_bytes = int(workspace_bytes)
    return d


def bwd(q, k, v, dout, log_alpha=None, *, log_ig=None, initial_state=None, dfinal_state=None, stream=None):
    """Gradients of the forward pass on the current HIP stream (every gate kind).

    ``dout`` [B,H,L,Dv] and ``dfinal_state`` [B,H,Dk,Dv] (or None) are fp32 loss gradients
    with respect to the outputs.  Returns a dict of fp32 tensors: ``dq``, ``dk``, ``dv``,
    ``dlog_alpha`` (layout of ``log_alpha``; None without a gate), ``dlog_ig`` (None without
    an input gate) and ``dinitial_state``."""
    import torch

    lib = load()
    _check_fwd_shapes(q, k, v, log_alpha, log_ig, initial_state, None, None)
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    _check_shape(dout, (B, H, L, Dv), "dout")
    _check_shape(dfinal_state, (B, H, Dk, Dv), "dfinal_state")
    f = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty((B, H, L, Dk), **f), torch.empty((B, H, L, Dk), **f), torch.empty((B, H, L, Dv), **f)
    dla = torch.empty(log_alpha.shape, **f) if log_alpha is not None else None
    dli = torch.empty((B, H, L), **f) if log_ig is not None else None
    ds0 = torch.empty((B, H, Dk, Dv), **f)
    _check_tensors(q, k, v, log_alpha, log_ig, initial_state, dout, dfinal_state, dq, dk, dv, dla, dli, ds0)
    d = make_bwd_desc(q, k, v, dout, dq, dk, dv, log_alpha, log_ig, initial_state, dfinal_state, dla, dli, ds0)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib.gla_bwd(ctypes.byref(d), ctypes.c_void_p(s.cuda_stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_bwd")
    return dict(dq=dq, dk=dk, dv=dv, dlog_alpha=dla, dlog_ig=dli, dinitial_state=ds0)


def fwd_headline(q, k, v, log_alpha, out, final_state, chunk: int = 64, stream=None) -> int:
    """The 13-argument entry point ``gla_fwd`` (bf16 inputs, per-channel gate or None); returns the status."""
    import torch

    if log_alpha is not None and log_alpha.dim() != 4:
        raise ValueError("gla_fwd takes a per-channel log_alpha [B, H, L, Dk] or None")
    _check_fwd_shapes(q, k, v, log_alpha, None, None, out, final_state)
    _check_tensors(q, k, v, log_alpha, out, final_state)
    if q.dtype != torch.bfloat16:
        raise TypeError("gla_fwd takes bf16 q, k, v")
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    return int(load().gla_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(out), _ptr(final_state), B, H, L,
                              Dk, Dv, int(chunk), ctypes.c_void_p(s.cuda_stream)))


def step_gate_kind_of(log_alpha, B: int, H: int, Dk: int) -> int:
    if log_alpha is None:
        return GATE_NONE
    shape = tuple(log_alpha.shape)
    if shape == (B, H, Dk):
        return GATE_CHANNEL
    if shape == (B, H):
        return GATE_HEAD
    if shape == (H,):
        return GATE_HEAD_CONST
    raise ValueError("log_alpha shape %s matches no gate layout for B=%d H=%d Dk=%d" % (shape, B, H, Dk))


def make_step_desc(q, k, v, state, out, log_alpha=None, log_ig=None, gate_kind=None) -> GlaStepDesc:
    """Fill a :class:`GlaStepDesc` (q, k: [B,H,Dk]; v: [B,H,Dv]; state [B,H,Dk,Dv])."""
    import torch

    B, H, Dk = q.shape
    Dv = v.shape[-1]
    d = GlaStepDesc()
    d.B, d.H, d.Dk, d.Dv = B, H, Dk, Dv
    if q.dtype == torch.bfloat16:
        d.in_dtype = DTYPE_BF16
    elif q.dtype == torch.float32:
        d.in_dtype = DTYPE_F32
    else:
        raise TypeError("q, k, v must be bf16 or fp32, got %s" % q.dtype)
    d.gate_kind = step_gate_kind_of(log_alpha, B, H, Dk) if gate_kind is None else int(gate_kind)
    d.q, d.k, d.v = _ptr(q), _ptr(k), _ptr(v)
    d.log_alpha, d.log_ig = _ptr(log_alpha), _ptr(log_ig)
    d.state, d.out = _ptr(state), _ptr(out)
    return d


def step(q, k, v, state, log_alpha=None, *, log_ig=None, out=None, stream=None):
    """One recurrent step on the current HIP stream: ``state`` [B,H,Dk,Dv] fp32 is updated in
    place (``S <- diag(alpha) S + i k^T v``) and ``o = q S`` [B,H,Dv] fp32 is returned."""
    import torch

    lib = load()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [B, H, D]")
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_shape(k, (B, H, Dk), "k")
    if log_alpha is not None:
        step_gate_kind_of(log_alpha, B, H, Dk)
    _check_shape(log_ig, (B, H), "log_ig")
    _check_shape(state, (B, H, Dk, Dv), "state")
    _check_shape(out, (B, H, Dv), "out")
    if out is None:
        out = torch.empty((B, H, Dv), dtype=torch.float32, device=q.device)
    _check_tensors(q, k, v, log_alpha, log_ig, state, out)
    d = make_step_desc(q, k, v, state, out, log_alpha, log_ig)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib.gla_step(ctypes.byref(d), ctypes.c_void_p(s.cuda_stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_step")
    return out


def plan(desc: GlaDesc) -> GlaPlan:
    p = GlaPlan()
    st = load().gla_query_plan(ctypes.byref(desc), ctypes.byref(p))
    if st != GLA_OK:
        raise GlaError(st, "gla_query_plan")
    return p


def workspace_size(desc: GlaDesc) -> int:
    n = ctypes.c_size_t(0)
    st = load().gla_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != GLA_OK:
        raise GlaError(st, "gla_workspace_size")
    return int(n.value)


# ---------------------------------------------------------------------------------------
# Delta rule (DeltaNet, Gated DeltaNet).

def delta_gate_kind_of(log_alpha, B: int, H: int, L: int) -> int:
    if log_alpha is None:
        return GATE_NONE
    shape = tuple(log_alpha.shape)
    if shape == (B, H, L):
        return GATE_HEAD
    if shape == (H,):
        return GATE_HEAD_CONST
    raise ValueError("log_alpha shape %s matches no delta-rule gate layout for B=%d H=%d L=%d" % (shape, B, H, L))


def make_delta_desc(q, k, v, beta, log_alpha=None, initial_state=None, out=None, final_state=None,
                    chunk=64, gate_kind=None) -> GlaDeltaDesc:
    """Fill a :class:`GlaDeltaDesc` from tensors (shapes read from q and v)."""
    import torch

    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    d = GlaDeltaDesc()
    d.B, d.H, d.L, d.Dk, d.Dv, d.chunk = B, H, L, Dk, Dv, int(chunk)
    if q.dtype == torch.bfloat16:
        d.in_dtype = DTYPE_BF16
    elif q.dtype == torch.float32:
        d.in_dtype = DTYPE_F32
    else:
        raise TypeError("q, k, v must be bf16 or fp32, got %s" % q.dtype)
    d.gate_kind = delta_gate_kind_of(log_alpha, B, H, L) if gate_kind is None else int(gate_kind)
    d.q, d.k, d.v, d.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(beta)
    d.log_alpha, d.initial_state = _ptr(log_alpha), _ptr(initial_state)
    d.out, d.final_state = _ptr(out), _ptr(final_state)
    return d


def delta_fwd(q, k, v, beta, log_alpha=None, *, initial_state=None, chunk: int = 64, final_state: bool = True,
              out=None, stream=None):
    """Delta-rule forward (``gla_delta_fwd``) on the current HIP stream: DeltaNet without
    ``log_alpha``, Gated DeltaNet with a ``[B,H,L]`` (or fixed ``[H]``) log decay.  ``beta``
    is the ``[B,H,L]`` fp32 writing strength.  Returns ``(out [B,H,L,Dv] fp32,
    final_state [B,H,Dk,Dv] fp32 or None)``."""
    import torch

    lib = load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, H, L, D]")
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    _check_shape(k, (B, H, L, Dk), "k")
    _check_shape(v, (B, H, L, Dv), "v")
    _check_shape(beta, (B, H, L), "beta")
    if log_alpha is not None:
        delta_gate_kind_of(log_alpha, B, H, L)
    _check_shape(initial_state, (B, H, Dk, Dv), "initial_state")
    _check_shape(out, (B, H, L, Dv), "out")
    if out is None:
        out = torch.empty((B, H, L, Dv), dtype=torch.float32, device=q.device)
    fin = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device) if final_state else None
    _check_tensors(q, k, v, beta, log_alpha, initial_state, out, fin)
    d = make_delta_desc(q, k, v, beta, log_alpha, initial_state, out, fin, chunk)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib.gla_delta_fwd(ctypes.byref(d), ctypes.c_void_p(s.cuda_stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_delta_fwd")
    return out, fin


def make_mlstm_desc(q, k, v, log_f, log_i, initial_state=None, out=None, final_state=None,
                    chunk=64) -> GlaMlstmDesc:
    """Fill a :class:`GlaMlstmDesc` from tensors (shapes read from q and v).  ``initial_state``
    and ``final_state`` are ``(C' [B,H,Dk,Dv], n' [B,H,Dk], m [B,H])`` triples or None."""
    import torch

    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    d = GlaMlstmDesc()
    d.B, d.H, d.L, d.Dk, d.Dv, d.chunk = B, H, L, Dk, Dv, int(chunk)
    if q.dtype == torch.bfloat16:
        d.in_dtype = DTYPE_BF16
    elif q.dtype == torch.float32:
        d.in_dtype = DTYPE_F32
    else:
        raise TypeError("q, k, v must be bf16 or fp32, got %s" % q.dtype)
    d.reserved = 0
    d.q, d.k, d.v, d.log_f, d.log_i = _ptr(q), _ptr(k), _ptr(v), _ptr(log_f), _ptr(log_i)
    if initial_state is not None:
        d.initial_C, d.initial_n, d.initial_m = (_ptr(t) for t in initial_state)
    d.out = _ptr(out)
    if final_state is not None:
        d.final_C, d.final_n, d.final_m = (_ptr(t) for t in final_state)
    return d


def mlstm_fwd(q, k, v, log_f, log_i, *, initial_state=None, chunk: int = 64, final_state: bool = True, out=None,
              stream=None):
    """mLSTM forward with exponential input gate and normaliser (``gla_mlstm_fwd``) on the
    current HIP stream.  ``log_f``, ``log_i``: ``[B,H,L]`` fp32 natural logs of the forget and
    input gates.  ``initial_state``: stabilised ``(C', n', m)`` or None.  Returns
    ``(out [B,H,L,Dv] fp32, (C', n', m) or None)`` with ``C = exp(m) C'``, ``n = exp(m) n'``."""
    import torch

    lib = load()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, H, L, D]")
    B, H, L, Dk = q.shape
    Dv = v.shape[-1]
    _check_shape(k, (B, H, L, Dk), "k")
    _check_shape(v, (B, H, L, Dv), "v")
    _check_shape(log_f, (B, H, L), "log_f")
    _check_shape(log_i, (B, H, L), "log_i")
    init = ()
    if initial_state is not None:
        if len(initial_state) != 3:
            raise ValueError("initial_state is a (C', n', m) triple")
        for t, shape, name in zip(initial_state, ((B, H, Dk, Dv), (B, H, Dk), (B, H)), ("C'", "n'", "m")):
            if t is None:
                raise ValueError("initial_state: %s missing" % name)
            _check_shape(t, shape, "initial " + name)
        init = tuple(initial_state)
    _check_shape(out, (B, H, L, Dv), "out")
    if out is None:
        out = torch.empty((B, H, L, Dv), dtype=torch.float32, device=q.device)
    fin = None
    if final_state:
        fin = (torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device),
               torch.empty((B, H, Dk), dtype=torch.float32, device=q.device),
               torch.empty((B, H), dtype=torch.float32, device=q.device))
    _check_tensors(q, k, v, log_f, log_i, out, *init, *(fin or ()))
    d = make_mlstm_desc(q, k, v, log_f, log_i, initial_state, out, fin, chunk)
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = lib.gla_mlstm_fwd(ctypes.byref(d), ctypes.c_void_p(s.cuda_stream))
    if st != GLA_OK:
        raise GlaError(st, "gla_mlstm_fwd")
    return out, fin
