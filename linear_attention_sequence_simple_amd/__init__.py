"""Python binding of libgla, the gfx950 Simple GLA mixer library.

Argument marshalling only: torch supplies device memory and the current HIP
stream, every step of the computation runs in the library's kernels.  The
functions carry the names of the C entry points (include/gla.h):

    gla_chunk_fwd(q, k, v, g, S0=None, out_dtype=None)        -> (o, S_T)
    gla_chunk_fwd_strided(q, k, v, g, S0=None, out_dtype=None, o=None, gate=None)
                                                               -> (o, S_T)
    gla_chunk_fwd_noalloc(q, k, v, g, o, S0=None, S_T=None)    -> (o, S_T)
    gla_chunk_fwd_varlen(q, k, v, g, cu_seqlens, max_seqlen, pool,
                         slot_idx=None, init_from_pool=False,
                         out_dtype=None)                       -> o
    gla_recurrent_step(pool, q, k, v, g, slot_idx=None, out_dtype=None) -> o
    gla_chunk_bwd(q, k, v, g, dO, S0=None, dS_T=None, out_dtype=None,
                  want_dS0=False)                             -> (dq, dk, dv, dg, dS0)
    gla_conv1d_silu(x, w, bias=None, conv_state=None, slot_idx=None,
                    init_from_state=False, cu_seqlens=None, max_seqlen=None,
                    out_dtype=None)                            -> y
    gla_state_alloc(n_slots, H=16, dk=96, dv=192)             -> StatePool
    gla_state_alloc_q16(n_slots, H=16, dk=96, dv=192)         -> StatePool (16-bit)
    gla_state_alloc_conv(n_slots, conv_D, H=16, dk=96, dv=192, fmt=GLA_STATE_F32)
                                                              -> StatePool with a conv window per slot
    gla_conv1d_silu_pool(x, w, pool, bias=None, slot_idx=None, init_from_pool=False,
                         cu_seqlens=None, max_seqlen=None, out_dtype=None) -> y
    gla_state_format(pool)                                    -> GLA_STATE_F32 | GLA_STATE_Q16
    gla_state_write(pool, S, slot_idx=None)                   (float32 states into slots)
    gla_state_read(pool, n=None, slot_idx=None, S=None)       -> S float32
    gla_workspace_size(op, dims)                              -> int

Layouts: q, k [B,T,H,96]; v, o, dO [B,T,H,192]; g [B,T,H] float32; states
[B,H,96,192] float32; packed sequences [N,H,...] with int32 offsets
cu_seqlens [n_seq+1] and their states in a StatePool.  There is no fallback: without the built library on a
GPU every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["GLA_F32", "GLA_BF16", "GLA_OP_FWD", "GLA_OP_BWD", "GLA_OP_FWD_VARLEN_Q16", "GlaError", "GlaDims",
           "lib", "lib_path", "gla_chunk_fwd", "gla_chunk_fwd_noalloc", "gla_chunk_fwd_strided", "gla_chunk_fwd_varlen", "gla_recurrent_step", "gla_chunk_bwd",
           "gla_conv1d_silu", "gla_conv1d_silu_pool", "gla_state_alloc_conv", "gla_state_alloc_q16",
           "gla_state_format", "gla_state_write",
           "gla_state_read", "GLA_STATE_F32", "GLA_STATE_Q16",
           "gla_state_alloc", "gla_workspace_size", "StatePool", "EXPORTS",
           "chunk_fwd", "recurrent_step", "chunk_bwd"]

GLA_F32, GLA_BF16 = 0, 1
GLA_OP_FWD, GLA_OP_BWD, GLA_OP_FWD_VARLEN_Q16 = 0, 1, 2
GLA_STATE_F32, GLA_STATE_Q16 = 0, 1
CHUNK, DK, DV = 128, 96, 192
STATUS = {0: "GLA_OK", 1: "GLA_ERR_INVALID_ARGUMENT", 2: "GLA_ERR_UNSUPPORTED",
          3: "GLA_ERR_OUT_OF_MEMORY", 4: "GLA_ERR_DEVICE"}
EXPORTS = ["gla_state_alloc", "gla_state_free", "gla_state_ptr", "gla_state_slots",
           "gla_state_slot_bytes", "gla_workspace_size", "gla_chunk_fwd",
           "gla_chunk_fwd_strided", "gla_chunk_fwd_varlen", "gla_recurrent_step", "gla_chunk_bwd",
           "gla_conv1d_silu", "gla_state_alloc_q16", "gla_state_format", "gla_state_q16_ptrs",
           "gla_state_write", "gla_state_read", "gla_status_str", "gla_last_error", "gla_chunk_fwd_noalloc",
           "gla_conv1d_silu_pool", "gla_state_alloc_conv", "gla_state_conv_channels", "gla_state_conv_ptr",
           "gla_state_seq_bytes"]


class GlaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class GlaDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32), ("segments", ctypes.c_int32)]


class GlaStrides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("token", ctypes.c_int64), ("head", ctypes.c_int64)]


_LIB = None


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgla.so")


def lib():
    """Load libgla.so (built in-tree by build.py) and declare its signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m linear_attention_sequence_simple_amd.build`")
    L = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.gla_state_alloc.argtypes = [I64, I32, I32, I32, P, ctypes.POINTER(P)]
    L.gla_state_free.argtypes = [P]
    L.gla_state_ptr.argtypes = [P, I64]
    L.gla_state_ptr.restype = P
    L.gla_state_slots.argtypes = [P]
    L.gla_state_slots.restype = I64
    L.gla_state_slot_bytes.argtypes = [I32, I32, I32]
    L.gla_state_slot_bytes.restype = SZ
    L.gla_workspace_size.argtypes = [I32, ctypes.POINTER(GlaDims), ctypes.POINTER(SZ)]
    L.gla_chunk_fwd.argtypes = [ctypes.POINTER(GlaDims), P, P, P, P, P, P, P, P, SZ, P]
    L.gla_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(GlaDims), P, P, P, P, P, P, P, P]
    SP = ctypes.POINTER(GlaStrides)
    L.gla_chunk_fwd_strided.argtypes = [ctypes.POINTER(GlaDims), P, SP, P, SP, P, SP, P, SP, P, SP, P, P, SP, P, P,
                                        SZ, P]
    L.gla_chunk_fwd_varlen.argtypes = [ctypes.POINTER(GlaDims), I64, P, P, P, P, P, P, P, I32, P, P, SZ, P]
    L.gla_recurrent_step.argtypes = [I64, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P]
    L.gla_chunk_bwd.argtypes = [ctypes.POINTER(GlaDims), P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
    L.gla_conv1d_silu.argtypes = [I64, I64, I32, I32, I32, P, I64, P, P, P, P, P, I32, P, P]
    L.gla_conv1d_silu_pool.argtypes = [I64, I64, I32, I32, P, I64, P, P, P, P, P, I32, P, P]
    L.gla_state_alloc_conv.argtypes = [I64, I32, I32, I32, I32, I32, P, ctypes.POINTER(P)]
    L.gla_state_conv_channels.argtypes = [P]
    L.gla_state_conv_channels.restype = I32
    L.gla_state_conv_ptr.argtypes = [P, I64]
    L.gla_state_conv_ptr.restype = P
    L.gla_state_seq_bytes.argtypes = [I32, I32, I32, I32, I32]
    L.gla_state_seq_bytes.restype = SZ
    L.gla_state_alloc_q16.argtypes = [I64, I32, I32, I32, P, ctypes.POINTER(P)]
    L.gla_state_format.argtypes = [P]
    L.gla_state_format.restype = I32
    L.gla_state_q16_ptrs.argtypes = [P, I64, ctypes.POINTER(P), ctypes.POINTER(P)]
    L.gla_state_write.argtypes = [P, I64, P, P, P]
    L.gla_state_read.argtypes = [P, I64, P, P, P]
    L.gla_status_str.argtypes = [I32]
    L.gla_status_str.restype = ctypes.c_char_p
    L.gla_last_error.restype = ctypes.c_char_p
    for name in ("gla_state_alloc", "gla_state_free", "gla_workspace_size", "gla_chunk_fwd", "gla_chunk_fwd_noalloc",
                 "gla_chunk_fwd_strided", "gla_chunk_fwd_varlen", "gla_recurrent_step", "gla_chunk_bwd",
                 "gla_conv1d_silu", "gla_conv1d_silu_pool", "gla_state_alloc_conv", "gla_state_alloc_q16",
                 "gla_state_q16_ptrs", "gla_state_write", "gla_state_read"):
        getattr(L, name).restype = I32
    _LIB = L
    return L


def _check(status):
    if status != 0:
        raise GlaError(status, lib().gla_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return GLA_F32
    if t == torch.bfloat16:
        return GLA_BF16
    raise TypeError(f"unsupported dtype {t}: use torch.float32 or torch.bfloat16")


def _torch_dtype(code: int) -> torch.dtype:
    return torch.float32 if code == GLA_F32 else torch.bfloat16


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dims(B, T, H, in_dtype, out_dtype, segments=None) -> GlaDims:
    """segments: None lets the library pick its launch plan; n > 0 splits every
    walk into n segments of whole chunks (the dims' one plan choice)."""
    return GlaDims(B, T, H, DK, DV, CHUNK, in_dtype, out_dtype, 0 if segments is None else int(segments))


def gla_workspace_size(op: int, dims: GlaDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().gla_workspace_size(op, ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace of {workspace.numel() * workspace.element_size()} B < {nbytes} B")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gla_chunk_fwd(q, k, v, g, S0=None, out_dtype=None, want_state=True, workspace=None, o=None,
                  S_T=None, segments=None):
    """Chunked prefill.  Returns (o, S_T); S_T is None when want_state is False."""
    B, T, H, _ = q.shape
    dev = q.device
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    _need(q, "q", (B, T, H, DK), q.dtype, dev)
    _need(k, "k", (B, T, H, DK), q.dtype, dev)
    _need(v, "v", (B, T, H, DV), q.dtype, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, DK, DV), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, DV), dtype=_torch_dtype(out_code), device=dev)
    _need(o, "o", (B, T, H, DV), _torch_dtype(out_code), dev)
    if want_state and S_T is None:
        S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need(S_T, "S_T", (B, H, DK, DV), torch.float32, dev)
    dims = _dims(B, T, H, in_code, out_code, segments)
    ws = _workspace(gla_workspace_size(GLA_OP_FWD, dims), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gla_chunk_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0),
                               _ptr(o), _ptr(S_T), _ptr(ws), nbytes, _stream()))
    return o, S_T


def gla_chunk_fwd_noalloc(q, k, v, g, o, S0=None, S_T=None, segments=None):
    """gla_chunk_fwd without a workspace and without any allocation: the
    caller passes o (and S_T, or None); a segmented plan uses the library's
    static scratch array.  Returns (o, S_T)."""
    B, T, H, _ = q.shape
    dev = q.device
    in_code = _dtype_code(q.dtype)
    out_code = _dtype_code(o.dtype)
    _need(q, "q", (B, T, H, DK), q.dtype, dev)
    _need(k, "k", (B, T, H, DK), q.dtype, dev)
    _need(v, "v", (B, T, H, DV), q.dtype, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    _need(o, "o", (B, T, H, DV), o.dtype, dev)
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None:
            _need(t, name, (B, H, DK, DV), torch.float32, dev)
    dims = _dims(B, T, H, in_code, out_code, segments)
    _check(lib().gla_chunk_fwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0),
                                       _ptr(o), _ptr(S_T), _stream()))
    return o, S_T


def _view_strides(t, name, shape, dtype, device):
    """Strides of a [B,T,H,d] (or [B,T,H]) view whose rows are contiguous."""
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    st = t.stride()
    if len(shape) == 4 and st[3] != 1:
        raise ValueError(f"{name} rows must be contiguous (last stride 1)")
    return GlaStrides(st[0], st[1], st[2])


def gla_chunk_fwd_strided(q, k, v, g, S0=None, out_dtype=None, want_state=True, workspace=None, o=None,
                          S_T=None, segments=None, gate=None):
    """gla_chunk_fwd on views with any positive batch/token/head strides (for
    example q, k, v sliced out of a fused projection output), rows contiguous.
    gate: None, or a [B,T,H,192] view in q's dtype; the output is then
    o * SiLU(gate), applied before the store."""
    B, T, H, _ = q.shape
    dev = q.device
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    sq = _view_strides(q, "q", (B, T, H, DK), q.dtype, dev)
    sk = _view_strides(k, "k", (B, T, H, DK), q.dtype, dev)
    sv = _view_strides(v, "v", (B, T, H, DV), q.dtype, dev)
    sg = _view_strides(g, "g", (B, T, H), torch.float32, dev)
    sgate = None if gate is None else _view_strides(gate, "gate", (B, T, H, DV), q.dtype, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, DK, DV), torch.float32, dev)
    if o is None:
        o = torch.empty((B, T, H, DV), dtype=_torch_dtype(out_code), device=dev)
    so = _view_strides(o, "o", (B, T, H, DV), _torch_dtype(out_code), dev)
    if want_state and S_T is None:
        S_T = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev)
    if S_T is not None:
        _need(S_T, "S_T", (B, H, DK, DV), torch.float32, dev)
    dims = _dims(B, T, H, in_code, out_code, segments)
    ws = _workspace(gla_workspace_size(GLA_OP_FWD, dims), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    r = ctypes.byref
    _check(lib().gla_chunk_fwd_strided(r(dims), _ptr(q), r(sq), _ptr(k), r(sk), _ptr(v), r(sv), _ptr(g), r(sg),
                                       _ptr(gate), None if sgate is None else r(sgate),
                                       _ptr(S0), _ptr(o), r(so), _ptr(S_T), _ptr(ws), nbytes, _stream()))
    return o, S_T


def gla_chunk_fwd_varlen(q, k, v, g, cu_seqlens, max_seqlen, pool, slot_idx=None,
                         init_from_pool=False, out_dtype=None, workspace=None, o=None, segments=None):
    """Prefill of packed sequences of different lengths into pool slots.

    q, k [N,H,96]; v [N,H,192]; g [N,H] float32; cu_seqlens int32 [n_seq+1]
    on the device (sequence b is rows cu_seqlens[b]:cu_seqlens[b+1]);
    max_seqlen bounds every sequence's length; pool a StatePool; slot_idx
    int32 [n_seq] on the device or None (sequence b uses slot b).  Each
    sequence starts from its slot's state (init_from_pool) or from zero, and
    its final state is written to the slot (encoded, for a 16-bit pool).
    Returns o [N,H,192].
    """
    N, H, _ = q.shape
    dev = q.device
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    _need(q, "q", (N, H, DK), q.dtype, dev)
    _need(k, "k", (N, H, DK), q.dtype, dev)
    _need(v, "v", (N, H, DV), q.dtype, dev)
    _need(g, "g", (N, H), torch.float32, dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-d tensor of n_seq + 1 offsets")
    n_seq = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", (n_seq + 1,), torch.int32, dev)
    if slot_idx is not None:
        _need(slot_idx, "slot_idx", (n_seq,), torch.int32, dev)
    if o is None:
        o = torch.empty((N, H, DV), dtype=_torch_dtype(out_code), device=dev)
    _need(o, "o", (N, H, DV), _torch_dtype(out_code), dev)
    dims = _dims(n_seq, int(max_seqlen), H, in_code, out_code, segments)
    op = GLA_OP_FWD_VARLEN_Q16 if pool.fmt == GLA_STATE_Q16 else GLA_OP_FWD
    ws = _workspace(gla_workspace_size(op, dims), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gla_chunk_fwd_varlen(ctypes.byref(dims), N, _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(g), pool.handle, _ptr(slot_idx), int(bool(init_from_pool)),
                                      _ptr(o), _ptr(ws), nbytes, _stream()))
    return o


def gla_chunk_bwd(q, k, v, g, dO, S0=None, dS_T=None, out_dtype=None, want_dS0=False,
                  workspace=None, segments=None):
    """Chunked backward.  Returns (dq, dk, dv, dg, dS0); dS0 is None unless want_dS0."""
    B, T, H, _ = q.shape
    dev = q.device
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    _need(q, "q", (B, T, H, DK), q.dtype, dev)
    _need(k, "k", (B, T, H, DK), q.dtype, dev)
    _need(v, "v", (B, T, H, DV), q.dtype, dev)
    _need(dO, "dO", (B, T, H, DV), q.dtype, dev)
    _need(g, "g", (B, T, H), torch.float32, dev)
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _need(t, name, (B, H, DK, DV), torch.float32, dev)
    od = _torch_dtype(out_code)
    dq = torch.empty((B, T, H, DK), dtype=od, device=dev)
    dk = torch.empty((B, T, H, DK), dtype=od, device=dev)
    dv = torch.empty((B, T, H, DV), dtype=od, device=dev)
    dg = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dS0 = torch.empty((B, H, DK, DV), dtype=torch.float32, device=dev) if want_dS0 else None
    dims = _dims(B, T, H, in_code, out_code, segments)
    ws = _workspace(gla_workspace_size(GLA_OP_BWD, dims), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().gla_chunk_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0),
                               _ptr(dO), _ptr(dS_T), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
                               _ptr(dS0), _ptr(ws), nbytes, _stream()))
    return dq, dk, dv, dg, dS0


def gla_conv1d_silu(x, w, bias=None, conv_state=None, slot_idx=None, init_from_state=False,
                    cu_seqlens=None, max_seqlen=None, out_dtype=None, y=None):
    """Causal depth-wise convolution of width 4 with SiLU.

    x [B,T,D] (or [N,D] with int32 cu_seqlens [n_seq+1] on the device and
    max_seqlen); w [D,4] float32; bias [D] float32 or None; conv_state
    [n_slots,4,D] float32 or None (each sequence's window of its last four
    inputs, updated in place); slot_idx int32 [n_seq] on the device or None.
    Returns y.
    """
    dev = x.device
    in_code = _dtype_code(x.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    D = x.shape[-1]
    if cu_seqlens is None:
        if x.dim() != 3:
            raise ValueError("x must be [B, T, D] without cu_seqlens")
        B, T = x.shape[0], x.shape[1]
        total = B * T
    else:
        if x.dim() != 2 or max_seqlen is None:
            raise ValueError("x must be [N, D] with cu_seqlens, and max_seqlen must be given")
        B, T, total = cu_seqlens.numel() - 1, int(max_seqlen), x.shape[0]
        _need(cu_seqlens, "cu_seqlens", (B + 1,), torch.int32, dev)
    _need(x, "x", tuple(x.shape), x.dtype, dev)
    _need(w, "w", (D, 4), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (D,), torch.float32, dev)
    if conv_state is not None:
        if conv_state.dim() != 3 or tuple(conv_state.shape[1:]) != (4, D):
            raise ValueError(f"conv_state must be [n_slots, 4, {D}]")
        _need(conv_state, "conv_state", tuple(conv_state.shape), torch.float32, dev)
    if slot_idx is not None:
        _need(slot_idx, "slot_idx", (B,), torch.int32, dev)
    if y is None:
        y = torch.empty(tuple(x.shape), dtype=_torch_dtype(out_code), device=dev)
    _need(y, "y", tuple(x.shape), _torch_dtype(out_code), dev)
    _check(lib().gla_conv1d_silu(B, T, D, in_code, out_code, _ptr(cu_seqlens), total, _ptr(x), _ptr(w),
                                 _ptr(bias), _ptr(conv_state), _ptr(slot_idx), int(bool(init_from_state)),
                                 _ptr(y), _stream()))
    return y


def gla_conv1d_silu_pool(x, w, pool, bias=None, slot_idx=None, init_from_pool=False, cu_seqlens=None,
                         max_seqlen=None, out_dtype=None, y=None):
    """gla_conv1d_silu with each sequence's window in its slot of `pool` (a
    StatePool made with conv_D); x has pool.conv_D channels."""
    dev = x.device
    in_code = _dtype_code(x.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    D = pool.conv_D
    if not D:
        raise ValueError("the pool has no convolution window (make it with gla_state_alloc_conv)")
    if x.shape[-1] != D:
        raise ValueError(f"x has {x.shape[-1]} channels, the pool's window {D}")
    if cu_seqlens is None:
        if x.dim() != 3:
            raise ValueError("x must be [B, T, D] without cu_seqlens")
        B, T, total = x.shape[0], x.shape[1], x.shape[0] * x.shape[1]
    else:
        if x.dim() != 2 or max_seqlen is None:
            raise ValueError("x must be [N, D] with cu_seqlens, and max_seqlen must be given")
        B, T, total = cu_seqlens.numel() - 1, int(max_seqlen), x.shape[0]
        _need(cu_seqlens, "cu_seqlens", (B + 1,), torch.int32, dev)
    _need(x, "x", tuple(x.shape), x.dtype, dev)
    _need(w, "w", (D, 4), torch.float32, dev)
    if bias is not None:
        _need(bias, "bias", (D,), torch.float32, dev)
    if slot_idx is not None:
        _need(slot_idx, "slot_idx", (B,), torch.int32, dev)
    if y is None:
        y = torch.empty(tuple(x.shape), dtype=_torch_dtype(out_code), device=dev)
    _need(y, "y", tuple(x.shape), _torch_dtype(out_code), dev)
    _check(lib().gla_conv1d_silu_pool(B, T, in_code, out_code, _ptr(cu_seqlens), total, _ptr(x), _ptr(w),
                                      _ptr(bias), pool.handle, _ptr(slot_idx), int(bool(init_from_pool)),
                                      _ptr(y), _stream()))
    return y


class _DeviceArray:
    """A device buffer described for torch.as_tensor (no copy)."""

    def __init__(self, ptr, shape, typestr):
        self.__cuda_array_interface__ = {"shape": shape, "typestr": typestr, "data": (ptr, False),
                                         "version": 3, "strides": None}


class StatePool:
    """A library-owned pool of recurrent states [n_slots, H, dk, dv]: float32
    (fmt GLA_STATE_F32) or 16-bit mantissas with one exponent per state column
    (GLA_STATE_Q16)."""

    def __init__(self, n_slots, H=16, dk=DK, dv=DV, fmt=GLA_STATE_F32, conv_D=0):
        handle = ctypes.c_void_p()
        if conv_D:
            _check(lib().gla_state_alloc_conv(n_slots, H, dk, dv, fmt, conv_D, _stream(), ctypes.byref(handle)))
        else:
            alloc = lib().gla_state_alloc_q16 if fmt == GLA_STATE_Q16 else lib().gla_state_alloc
            _check(alloc(n_slots, H, dk, dv, _stream(), ctypes.byref(handle)))
        self._h = handle
        self.n_slots, self.H, self.dk, self.dv = n_slots, H, dk, dv
        self.fmt = lib().gla_state_format(handle)
        self.conv_D = lib().gla_state_conv_channels(handle)
        self.device = torch.device("cuda", torch.cuda.current_device())

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("the pool has been freed")
        return self._h

    def ptr(self, slot=0) -> int:
        if self.fmt != GLA_STATE_F32:
            raise TypeError("a 16-bit pool has no float32 slots: use q16_views() or gla_state_read")
        p = lib().gla_state_ptr(self.handle, slot)
        if not p:
            raise IndexError(f"slot {slot} out of range [0, {self.n_slots})")
        return p

    @property
    def slot_bytes(self) -> int:
        return lib().gla_state_slot_bytes(self.H, self.dk, self.dv)

    @property
    def __cuda_array_interface__(self):
        if self.fmt != GLA_STATE_F32:
            raise TypeError("a 16-bit pool has no float32 view: use q16_views() or gla_state_read")
        return {"shape": (self.n_slots, self.H, self.dk, self.dv), "typestr": "<f4",
                "data": (self.ptr(0), False), "version": 3, "strides": None}

    def view(self) -> torch.Tensor:
        """A torch tensor aliasing a float32 pool (no copy)."""
        if self.fmt != GLA_STATE_F32:
            raise TypeError("a 16-bit pool has no float32 view: use q16_views() or gla_state_read")
        return torch.as_tensor(self, device=self.device)

    def conv_view(self) -> torch.Tensor:
        """The convolution windows [n_slots, 4, conv_D] float32 (no copy)."""
        if not self.conv_D:
            raise TypeError("the pool has no convolution window")
        p = lib().gla_state_conv_ptr(self.handle, 0)
        arr = _DeviceArray(p, (self.n_slots, 4, self.conv_D), "<f4")
        return torch.as_tensor(arr, device=self.device)

    @property
    def seq_bytes(self) -> int:
        """Bytes of one slot: the mixer state and the convolution window."""
        return lib().gla_state_seq_bytes(self.H, self.dk, self.dv, self.fmt, self.conv_D)

    def q16_views(self):
        """(mantissas int16 [n_slots,H,dk,dv], exponents int32 [n_slots,H,dv])
        aliasing a 16-bit pool (no copy)."""
        m, e = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().gla_state_q16_ptrs(self.handle, 0, ctypes.byref(m), ctypes.byref(e)))
        mant = _DeviceArray(m.value, (self.n_slots, self.H, self.dk, self.dv), "<i2")
        expo = _DeviceArray(e.value, (self.n_slots, self.H, self.dv), "<i4")
        return torch.as_tensor(mant, device=self.device), torch.as_tensor(expo, device=self.device)

    def free(self):
        if self._h is not None:
            _check(lib().gla_state_free(self._h))
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def gla_state_alloc(n_slots, H=16, dk=DK, dv=DV) -> StatePool:
    return StatePool(n_slots, H, dk, dv)


def gla_state_alloc_q16(n_slots, H=16, dk=DK, dv=DV) -> StatePool:
    return StatePool(n_slots, H, dk, dv, fmt=GLA_STATE_Q16)


def gla_state_alloc_conv(n_slots, conv_D, H=16, dk=DK, dv=DV, fmt=GLA_STATE_F32) -> StatePool:
    """A pool whose slots hold a layer's mixer state (float32 or 16-bit) and
    its convolution window [4, conv_D] float32."""
    return StatePool(n_slots, H, dk, dv, fmt=fmt, conv_D=conv_D)


def gla_state_format(pool: StatePool) -> int:
    return lib().gla_state_format(pool.handle)


def gla_state_write(pool: StatePool, S, slot_idx=None):
    """Float32 states S [n,H,dk,dv] into slots slot_idx (int32 [n]) or 0..n-1
    (encoded for a 16-bit pool)."""
    n = S.shape[0]
    _need(S, "S", (n, pool.H, pool.dk, pool.dv), torch.float32, pool.device)
    if slot_idx is not None:
        _need(slot_idx, "slot_idx", (n,), torch.int32, pool.device)
    _check(lib().gla_state_write(pool.handle, n, _ptr(slot_idx), _ptr(S), _stream()))


def gla_state_read(pool: StatePool, n=None, slot_idx=None, S=None) -> torch.Tensor:
    """Float32 states of slots slot_idx (int32 [n]) or 0..n-1 (decoded from a
    16-bit pool), as S [n,H,dk,dv]."""
    if n is None:
        n = pool.n_slots if slot_idx is None else slot_idx.shape[0]
    if slot_idx is not None:
        _need(slot_idx, "slot_idx", (n,), torch.int32, pool.device)
    if S is None:
        S = torch.empty((n, pool.H, pool.dk, pool.dv), dtype=torch.float32, device=pool.device)
    _need(S, "S", (n, pool.H, pool.dk, pool.dv), torch.float32, pool.device)
    _check(lib().gla_state_read(pool.handle, n, _ptr(slot_idx), _ptr(S), _stream()))
    return S


def gla_recurrent_step(pool: StatePool, q, k, v, g, slot_idx=None, out_dtype=None, o=None):
    """One decode token per sequence; updates the pool in place and returns o [B,H,dv]."""
    B, H, _ = q.shape
    dev = q.device
    in_code = _dtype_code(q.dtype)
    out_code = in_code if out_dtype is None else _dtype_code(out_dtype)
    _need(q, "q", (B, H, DK), q.dtype, dev)
    _need(k, "k", (B, H, DK), q.dtype, dev)
    _need(v, "v", (B, H, DV), q.dtype, dev)
    _need(g, "g", (B, H), torch.float32, dev)
    if slot_idx is not None:
        _need(slot_idx, "slot_idx", (B,), torch.int32, dev)
    if o is None:
        o = torch.empty((B, H, DV), dtype=_torch_dtype(out_code), device=dev)
    _need(o, "o", (B, H, DV), _torch_dtype(out_code), dev)
    _check(lib().gla_recurrent_step(B, H, DK, DV, in_code, out_code, _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(g), pool.handle, _ptr(slot_idx), _ptr(o), _stream()))
    return o


# Short names: the three calls of the mixer without the C prefix.
chunk_fwd = gla_chunk_fwd
recurrent_step = gla_recurrent_step


def chunk_bwd(q, k, v, g, dO, S0=None, dS_T=None, **kw):
    """gla_chunk_bwd returning (dq, dk, dv, dg), followed by dS0 when an
    initial state is given (or want_dS0=True is passed)."""
    want = kw.pop("want_dS0", S0 is not None)
    r = gla_chunk_bwd(q, k, v, g, dO, S0, dS_T, want_dS0=want, **kw)
    return r if want else r[:4]
