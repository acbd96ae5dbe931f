"""Thin Python binding of the C ABI in include/gdn2.h (argument marshalling only).

``chunk_fwd``, ``chunk_bwd`` and ``recurrent_step`` take torch CUDA (HIP) tensors, check
dtype / shape / device / contiguity, and pass raw device pointers plus
torch's current stream to ``libgdn2.so``.  Every step of the computation runs
in the library's gfx950 kernels; there is no CPU or torch fallback: if the
library is missing or a call fails, these functions raise.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgdn2.so")

GDN2_F32, GDN2_BF16 = 0, 1
GDN2_GATE_HEAD, GDN2_GATE_KEY = 0, 1
GDN2_FORM_KEY, GDN2_FORM_VALUE_WRITE = 0, 1
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_UNSUPPORTED",
          5: "ERR_ALIAS", 6: "ERR_WORKSPACE", 7: "ERR_HIP", 8: "ERR_SCRATCH"}

# Every entry point include/gdn2.h declares.
EXPORTS = ("gdn2_abi_version", "gdn2_status_str", "gdn2_chunk_fwd_workspace",
           "gdn2_chunk_fwd", "gdn2_chunk_fwd_static", "gdn2_chunk_fwd_varlen_workspace", "gdn2_chunk_fwd_varlen",
           "gdn2_chunk_bwd_workspace", "gdn2_chunk_bwd", "gdn2_chunk_bwd_varlen_workspace",
           "gdn2_chunk_bwd_varlen", "gdn2_recurrent_step")


class Gdn2Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("chunk", ctypes.c_int64),
        ("qkv_dtype", ctypes.c_int32), ("decay_kind", ctypes.c_int32),
        ("erase_kind", ctypes.c_int32), ("write_kind", ctypes.c_int32),
        ("tie_write_to_erase", ctypes.c_int32), ("q_scale", ctypes.c_float),
        ("form", ctypes.c_int32), ("gate_logits", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
    ]


class Gdn2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_status_str(status)})")


_lock = threading.Lock()
_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libgdn2.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise ImportError(
                    f"{_LIB_PATH} is missing: build it with "
                    "`python -m gated_delta_rule_decay_amd.build`")
            lib = ctypes.CDLL(_LIB_PATH)
            vp, fp = ctypes.c_void_p, ctypes.c_void_p
            dp = ctypes.POINTER(Gdn2Desc)
            lib.gdn2_abi_version.restype = ctypes.c_int
            lib.gdn2_abi_version.argtypes = []
            lib.gdn2_status_str.restype = ctypes.c_char_p
            lib.gdn2_status_str.argtypes = [ctypes.c_int]
            lib.gdn2_chunk_fwd_workspace.restype = ctypes.c_int
            lib.gdn2_chunk_fwd_workspace.argtypes = [dp, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn2_chunk_fwd.restype = ctypes.c_int
            lib.gdn2_chunk_fwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp,
                                           ctypes.c_size_t, vp]
            lib.gdn2_chunk_fwd_static.restype = ctypes.c_int
            lib.gdn2_chunk_fwd_static.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp]
            lib.gdn2_chunk_fwd_varlen_workspace.restype = ctypes.c_int
            lib.gdn2_chunk_fwd_varlen_workspace.argtypes = [dp, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn2_chunk_fwd_varlen.restype = ctypes.c_int
            lib.gdn2_chunk_fwd_varlen.argtypes = [dp, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, vp,
                                                  ctypes.c_size_t, vp]
            lib.gdn2_chunk_bwd_workspace.restype = ctypes.c_int
            lib.gdn2_chunk_bwd_workspace.argtypes = [dp, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn2_chunk_bwd.restype = ctypes.c_int
            lib.gdn2_chunk_bwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                           fp, fp, fp, vp, ctypes.c_size_t, vp]
            lib.gdn2_chunk_bwd_varlen_workspace.restype = ctypes.c_int
            lib.gdn2_chunk_bwd_varlen_workspace.argtypes = [dp, ctypes.POINTER(ctypes.c_size_t)]
            lib.gdn2_chunk_bwd_varlen.restype = ctypes.c_int
            lib.gdn2_chunk_bwd_varlen.argtypes = [dp, vp, vp, vp, vp, fp, fp, fp, fp, fp, fp, fp, fp, fp, fp,
                                                  fp, fp, fp, vp, ctypes.c_size_t, vp]
            lib.gdn2_recurrent_step.restype = ctypes.c_int
            lib.gdn2_recurrent_step.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, fp, vp]
            _lib = lib
    return _lib


def _status_str(status: int) -> str:
    try:
        return load_library().gdn2_status_str(int(status)).decode()
    except Exception:  # pragma: no cover
        return "?"


def abi_version() -> int:
    return int(load_library().gdn2_abi_version())


def make_desc(batch, seqlen, heads, dk, dv, chunk=64, qkv_dtype=GDN2_BF16,
              decay_kind=GDN2_GATE_KEY, erase_kind=GDN2_GATE_KEY, write_kind=GDN2_GATE_KEY,
              tied=False, q_scale=1.0, form=GDN2_FORM_KEY, gate_logits=False,
              qk_l2norm=False, o_dtype=GDN2_F32) -> Gdn2Desc:
    return Gdn2Desc(batch, seqlen, heads, dk, dv, chunk, qkv_dtype, decay_kind, erase_kind,
                    write_kind, 1 if tied else 0, q_scale, form, int(bool(gate_logits)),
                    int(bool(qk_l2norm)), o_dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t, name, shape, dtypes, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gate_kind(g, tok_shape, dk, name):
    if g.dim() == len(tok_shape) + 1 and g.shape[-1] == dk:
        return GDN2_GATE_KEY, tuple(tok_shape) + (dk,)
    if g.dim() == len(tok_shape):
        return GDN2_GATE_HEAD, tuple(tok_shape)
    raise ValueError(f"{name} shape {tuple(g.shape)} is neither {tuple(tok_shape) + (dk,)} "
                     f"nor {tuple(tok_shape)}")


def _out_dtype(out, out_dtype):
    """The output's torch dtype and its gdn2_dtype: that of `out` when given,
    else `out_dtype` (default float32)."""
    import torch
    dt = out.dtype if out is not None else (out_dtype or torch.float32)
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"o must be float32 or bfloat16, not {dt}")
    return dt, (GDN2_BF16 if dt == torch.bfloat16 else GDN2_F32)


def _desc_for(q, k, v, log_decay, erase, write, tok_shape, batch, seqlen, heads, chunk, q_scale,
              value_write=False, qk_l2norm=False, o_dtype=GDN2_F32):
    import torch
    dk, dv = k.shape[-1], v.shape[-1]
    dev = k.device
    if k.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q/k/v must be bfloat16 or float32")
    for t, n, d in ((q, "q", dk), (k, "k", dk), (v, "v", dv)):
        _check(t, n, tuple(tok_shape) + (d,), (k.dtype,), dev)
    la_kind, la_shape = _gate_kind(log_decay, tok_shape, dk, "log_decay")
    eb_kind, eb_shape = _gate_kind(erase, tok_shape, dk, "erase")
    # fp32 gates, or bf16 logits that the kernels activate
    gate_logits = log_decay.dtype == torch.bfloat16
    gdt = (torch.bfloat16,) if gate_logits else (torch.float32,)
    _check(log_decay, "log_decay", la_shape, gdt, dev)
    _check(erase, "erase", eb_shape, gdt, dev)
    wr_kind = eb_kind
    if value_write and write is None:
        raise ValueError("the value-write form needs a write gate")
    if write is not None:
        # the value-write form gates the value channels
        wr_kind, wr_shape = _gate_kind(write, tok_shape, dv if value_write else dk, "write")
        _check(write, "write", wr_shape, gdt, dev)
    return make_desc(batch, seqlen, heads, dk, dv, chunk,
                     GDN2_BF16 if k.dtype == torch.bfloat16 else GDN2_F32,
                     la_kind, eb_kind, wr_kind, write is None, q_scale,
                     GDN2_FORM_VALUE_WRITE if value_write else GDN2_FORM_KEY, gate_logits, qk_l2norm, o_dtype)


def chunk_fwd_workspace(desc: Gdn2Desc) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().gdn2_chunk_fwd_workspace(ctypes.byref(desc), ctypes.byref(n))
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_fwd_workspace")
    return int(n.value)


def chunk_fwd(q, k, v, log_decay, erase, write=None, state0=None, chunk=64, q_scale=1.0,
              out=None, state_out=None, return_state=True, workspace=True, value_write=False,
              qk_l2norm=False, out_dtype=None):
    """Chunkwise GDN-2 forward on the GPU.

    q, k [B,T,H,dk], v [B,T,H,dv] (bf16 or fp32, one dtype); gates fp32
    [B,T,H,dk] or [B,T,H]; write None ties it to erase; state0 [B,H,dk,dv]
    fp32 or None.  ``workspace``: True allocates the two-pass scratch when
    the request has a two-pass kernel, False runs in one pass, or a uint8
    device tensor of at least chunk_fwd_workspace() bytes to use.
    ``value_write``: the gist.science form of the update (write gate
    [B,T,H,dv] or [B,T,H], required).  Gates given as bfloat16 tensors are
    raw logits (log a = -softplus, b and w = sigmoid, applied in-kernel);
    ``qk_l2norm`` normalises q and k per token-head in-kernel.  The output is
    fp32, or bf16 (the fp32 result rounded to nearest even) when ``out`` is a
    bfloat16 tensor or ``out_dtype`` is torch.bfloat16.
    Returns (o [B,T,H,dv], final state or None).
    """
    import torch
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    odt, o_code = _out_dtype(out, out_dtype)
    desc = _desc_for(q, k, v, log_decay, erase, write, (B, T, H), B, T, H, chunk, q_scale, value_write,
                     qk_l2norm, o_code)
    dev = k.device
    if state0 is not None:
        _check(state0, "state0", (B, H, dk, dv), (torch.float32,), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=odt, device=dev)
    else:
        _check(out, "out", (B, T, H, dv), (odt,), dev)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif state_out is not None:
        _check(state_out, "state_out", (B, H, dk, dv), (torch.float32,), dev)
    ws, ws_bytes = None, 0
    if workspace is True:
        ws_bytes = chunk_fwd_workspace(desc)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    elif workspace is not False and workspace is not None:
        _check(workspace, "workspace", tuple(workspace.shape), (torch.uint8,), dev)
        ws, ws_bytes = workspace, workspace.numel()
    st = load_library().gdn2_chunk_fwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase),
        _ptr(write), _ptr(state0), _ptr(out), _ptr(state_out), _ptr(ws), ws_bytes, _stream())
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_fwd")
    return out, state_out


def chunk_fwd_static(q, k, v, log_decay, erase, write=None, state0=None, chunk=64, q_scale=1.0,
                     out=None, state_out=None, return_state=True, value_write=False, qk_l2norm=False,
                     out_dtype=None):
    """``chunk_fwd`` through gdn2_chunk_fwd_static: the library's static
    device scratch instead of a workspace.  Allocates nothing when ``out``
    (and, with ``return_state``, ``state_out``) are given."""
    import torch
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    odt, o_code = _out_dtype(out, out_dtype)
    desc = _desc_for(q, k, v, log_decay, erase, write, (B, T, H), B, T, H, chunk, q_scale, value_write,
                     qk_l2norm, o_code)
    dev = k.device
    if state0 is not None:
        _check(state0, "state0", (B, H, dk, dv), (torch.float32,), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=odt, device=dev)
    else:
        _check(out, "out", (B, T, H, dv), (odt,), dev)
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif state_out is not None:
        _check(state_out, "state_out", (B, H, dk, dv), (torch.float32,), dev)
    st = load_library().gdn2_chunk_fwd_static(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase),
        _ptr(write), _ptr(state0), _ptr(out), _ptr(state_out), _stream())
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_fwd_static")
    return out, state_out


def chunk_fwd_varlen_workspace(desc: Gdn2Desc) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().gdn2_chunk_fwd_varlen_workspace(ctypes.byref(desc), ctypes.byref(n))
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_fwd_varlen_workspace")
    return int(n.value)


def chunk_fwd_varlen(q, k, v, log_decay, erase, write, cu_seqlens, state0=None, chunk=64,
                     q_scale=1.0, out=None, state_out=None, return_state=True, workspace=True,
                     value_write=False, qk_l2norm=False, out_dtype=None):
    """Chunkwise GDN-2 forward over N sequences packed along one token axis.

    q, k [T,H,dk], v [T,H,dv], gates [T,H,dk] / [T,H] (or the same with a
    leading 1); cu_seqlens int32 [N+1] on the device (sequence i is tokens
    cu_seqlens[i] .. cu_seqlens[i+1]-1); state0 [N,H,dk,dv] fp32 or None.
    Other arguments as for chunk_fwd.  Returns (o shaped like v but fp32,
    final states [N,H,dk,dv] or None).
    """
    import torch
    lead = k.shape[:-3]
    if len(lead) > 1 or (len(lead) == 1 and lead[0] != 1):
        raise ValueError("packed tensors are [T,H,d] or [1,T,H,d]")
    T, H, dk = k.shape[-3:]
    dv = v.shape[-1]
    dev = k.device
    _check(cu_seqlens, "cu_seqlens", tuple(cu_seqlens.shape), (torch.int32,), dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    odt, o_code = _out_dtype(out, out_dtype)
    desc = _desc_for(q, k, v, log_decay, erase, write, tuple(lead) + (T, H), N, T, H, chunk, q_scale,
                     value_write, qk_l2norm, o_code)
    if state0 is not None:
        _check(state0, "state0", (N, H, dk, dv), (torch.float32,), dev)
    oshape = tuple(lead) + (T, H, dv)
    if out is None:
        out = torch.empty(oshape, dtype=odt, device=dev)
    else:
        _check(out, "out", oshape, (odt,), dev)
    if state_out is None and return_state:
        state_out = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif state_out is not None:
        _check(state_out, "state_out", (N, H, dk, dv), (torch.float32,), dev)
    ws, ws_bytes = None, 0
    if workspace is True:
        ws_bytes = chunk_fwd_varlen_workspace(desc)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    elif workspace is not False and workspace is not None:
        _check(workspace, "workspace", tuple(workspace.shape), (torch.uint8,), dev)
        ws, ws_bytes = workspace, workspace.numel()
    st = load_library().gdn2_chunk_fwd_varlen(
        ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay),
        _ptr(erase), _ptr(write), _ptr(state0), _ptr(out), _ptr(state_out), _ptr(ws), ws_bytes,
        _stream())
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_fwd_varlen")
    return out, state_out


def chunk_bwd_workspace(desc: Gdn2Desc) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().gdn2_chunk_bwd_workspace(ctypes.byref(desc), ctypes.byref(n))
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_bwd_workspace")
    return int(n.value)


def chunk_bwd(q, k, v, log_decay, erase, write, state0, d_o, d_state=None, chunk=64,
              q_scale=1.0, want_state0=True, workspace=None, value_write=False, qk_l2norm=False):
    """Gradients of <d_o, o> + <d_state, S_T> for the chunkwise forward.

    Inputs as for ``chunk_fwd`` (``value_write``, bf16 gate logits and
    ``qk_l2norm`` included: the gradients are then those of the logits and
    of the raw q, k); d_o [B,T,H,dv] fp32; d_state [B,H,dk,dv] fp32 or None
    (zeros).  Returns a dict of fp32 tensors: dq, dk, dv, d_log_decay,
    d_erase, d_write (None when tied) shaped like their inputs, and d_state0
    (None unless ``want_state0``).  ``workspace``: None allocates it, or a
    uint8 device tensor of at least chunk_bwd_workspace() bytes.
    """
    import torch
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    desc = _desc_for(q, k, v, log_decay, erase, write, (B, T, H), B, T, H, chunk, q_scale, value_write,
                     qk_l2norm)
    dev = k.device
    f32 = (torch.float32,)
    if state0 is not None:
        _check(state0, "state0", (B, H, dk, dv), f32, dev)
    _check(d_o, "d_o", (B, T, H, dv), f32, dev)
    if d_state is not None:
        _check(d_state, "d_state", (B, H, dk, dv), f32, dev)
    new = lambda t: torch.empty(tuple(t.shape), dtype=torch.float32, device=dev)  # fp32 whatever t's dtype
    g = dict(dq=new(q), dk=new(k), dv=new(v), d_log_decay=new(log_decay), d_erase=new(erase),
             d_write=None if write is None else new(write),
             d_state0=torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_state0 else None)
    if workspace is None:
        n = chunk_bwd_workspace(desc)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", tuple(workspace.shape), (torch.uint8,), dev)
    st = load_library().gdn2_chunk_bwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase), _ptr(write),
        _ptr(state0), _ptr(d_o), _ptr(d_state), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
        _ptr(g["d_log_decay"]), _ptr(g["d_erase"]), _ptr(g["d_write"]), _ptr(g["d_state0"]),
        _ptr(workspace), workspace.numel(), _stream())
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_bwd")
    return g


def chunk_bwd_varlen_workspace(desc: Gdn2Desc) -> int:
    n = ctypes.c_size_t(0)
    st = load_library().gdn2_chunk_bwd_varlen_workspace(ctypes.byref(desc), ctypes.byref(n))
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_bwd_varlen_workspace")
    return int(n.value)


def chunk_bwd_varlen(q, k, v, log_decay, erase, write, cu_seqlens, state0, d_o, d_state=None, chunk=64,
                     q_scale=1.0, want_state0=True, workspace=None, value_write=False, qk_l2norm=False):
    """Gradients of the packed-sequence forward (``chunk_fwd_varlen``).

    Packed tensors [T,H,d] (or [1,T,H,d]) as for ``chunk_fwd_varlen``;
    cu_seqlens int32 [N+1] on the device; state0, d_state [N,H,dk,dv] fp32
    (or None); d_o shaped like v, fp32.  Returns the dict of ``chunk_bwd``
    (gradients shaped like their inputs, d_state0 [N,H,dk,dv]).
    """
    import torch
    lead = k.shape[:-3]
    if len(lead) > 1 or (len(lead) == 1 and lead[0] != 1):
        raise ValueError("packed tensors are [T,H,d] or [1,T,H,d]")
    T, H, dk = k.shape[-3:]
    dv = v.shape[-1]
    dev = k.device
    _check(cu_seqlens, "cu_seqlens", tuple(cu_seqlens.shape), (torch.int32,), dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D tensor of N+1 offsets")
    N = cu_seqlens.numel() - 1
    desc = _desc_for(q, k, v, log_decay, erase, write, tuple(lead) + (T, H), N, T, H, chunk, q_scale,
                     value_write, qk_l2norm)
    f32 = (torch.float32,)
    if state0 is not None:
        _check(state0, "state0", (N, H, dk, dv), f32, dev)
    _check(d_o, "d_o", tuple(lead) + (T, H, dv), f32, dev)
    if d_state is not None:
        _check(d_state, "d_state", (N, H, dk, dv), f32, dev)
    new = lambda t: torch.empty(tuple(t.shape), dtype=torch.float32, device=dev)  # fp32 whatever t's dtype
    g = dict(dq=new(q), dk=new(k), dv=new(v), d_log_decay=new(log_decay), d_erase=new(erase),
             d_write=None if write is None else new(write),
             d_state0=torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if want_state0 else None)
    if workspace is None:
        n = chunk_bwd_varlen_workspace(desc)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    else:
        _check(workspace, "workspace", tuple(workspace.shape), (torch.uint8,), dev)
    st = load_library().gdn2_chunk_bwd_varlen(
        ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase),
        _ptr(write), _ptr(state0), _ptr(d_o), _ptr(d_state), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
        _ptr(g["d_log_decay"]), _ptr(g["d_erase"]), _ptr(g["d_write"]), _ptr(g["d_state0"]),
        _ptr(workspace), workspace.numel(), _stream())
    if st != 0:
        raise Gdn2Error(st, "gdn2_chunk_bwd_varlen")
    return g


def recurrent_step(q, k, v, log_decay, erase, write, state, q_scale=1.0, out=None, value_write=False,
                   qk_l2norm=False, out_dtype=None):
    """One decode step for N sequences; updates ``state`` [N,H,dk,dv] in place.

    q, k [N,H,dk], v [N,H,dv]; gates [N,H,dk] or [N,H]; write None = tied.
    Returns o [N,H,dv], fp32 or (``out`` / ``out_dtype`` bfloat16) bf16.
    """
    import torch
    N, H, dk = k.shape
    dv = v.shape[-1]
    odt, o_code = _out_dtype(out, out_dtype)
    desc = _desc_for(q, k, v, log_decay, erase, write, (N, H), N, 1, H, 64, q_scale, value_write, qk_l2norm,
                     o_code)
    _check(state, "state", (N, H, dk, dv), (torch.float32,), k.device)
    if out is None:
        out = torch.empty((N, H, dv), dtype=odt, device=k.device)
    else:
        _check(out, "out", (N, H, dv), (odt,), k.device)
    st = load_library().gdn2_recurrent_step(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase),
        _ptr(write), _ptr(state), _ptr(out), _stream())
    if st != 0:
        raise Gdn2Error(st, "gdn2_recurrent_step")
    return out
