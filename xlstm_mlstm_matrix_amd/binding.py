"""Python binding of the C ABI in ``include/mlstm.h`` (ctypes).

Argument marshalling only: tensors are torch device tensors (torch supplies
device memory and the current stream); every step of the computation runs in
the HIP library.  There is no fallback: if ``libmlstm.so`` is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmlstm.so")

F32, BF16 = 0, 1
VARIANTS = {"auto": 0, "fused": 1, "segscan": 2}
STATUS = {0: "MLSTM_OK", 1: "MLSTM_ERR_NULL", 2: "MLSTM_ERR_SHAPE", 3: "MLSTM_ERR_UNSUPPORTED",
          4: "MLSTM_ERR_STATE_ARGS", 5: "MLSTM_ERR_WORKSPACE", 6: "MLSTM_ERR_ALIAS",
          7: "MLSTM_ERR_HIP", 8: "MLSTM_ERR_ALIGN", 9: "MLSTM_ERR_BLAS", 10: "MLSTM_ERR_SCRATCH"}
# bytes of the fixed per-device scratch of mlstm_step_noalloc (MLSTM_STEP_NOALLOC_MAX_BYTES)
STEP_NOALLOC_MAX_BYTES = 32 << 20

# exported entry points and their C signatures (kept in step with include/mlstm.h)
_vp, _fp, _sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
_i = ctypes.c_int
SIGNATURES = {
    "mlstm_status_string": (ctypes.c_char_p, [_i]),
    "mlstm_version": (ctypes.c_char_p, []),
    "mlstm_fwd_chunkwise_workspace_size": (_i, [_i] * 7 + [ctypes.POINTER(_sz)]),
    "mlstm_fwd_chunkwise_workspace_size_variant": (_i, [_i] * 8 + [ctypes.POINTER(_sz)]),
    "mlstm_fwd_chunkwise_schedule": (_i, [_i] * 8 + [ctypes.POINTER(_i)] * 2),
    "mlstm_fwd_chunkwise": (_i, [_vp] * 13 + [_i] * 7 + [_vp, _sz, _vp]),
    "mlstm_fwd_chunkwise_variant": (_i, [_vp] * 13 + [_i] * 8 + [_vp, _sz, _vp]),
    "mlstm_step_workspace_size": (_i, [_i] * 5 + [ctypes.POINTER(_sz)]),
    "mlstm_step": (_i, [_vp] * 13 + [_i] * 5 + [_vp, _sz, _vp]),
    "mlstm_step_noalloc": (_i, [_vp] * 13 + [_i] * 5 + [_vp]),
    "mlstm_bwd_chunkwise_workspace_size": (_i, [_i] * 7 + [ctypes.POINTER(_sz)]),
    "mlstm_bwd_chunkwise": (_i, [_vp] * 19 + [_i] * 7 + [_vp, _sz, _vp]),
    "mlstm_layer_fwd_workspace_size": (_i, [_i] * 8 + [ctypes.POINTER(_sz)]),
    "mlstm_layer_fwd": (_i, [_vp] * 20 + [_i] * 8 + [_vp, _sz, _vp]),
    "mlstm_slstm_fwd": (_i, [_vp] * 11 + [_i] * 5 + [_vp]),
}


class MlstmError(RuntimeError):
    """A non-OK status returned by the library."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} "
                               "(run python -m xlstm_mlstm_matrix_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_string(s: int) -> str:
    return lib().mlstm_status_string(int(s)).decode()


def _check(s: int):
    if s != 0:
        raise MlstmError(s, status_string(s))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _io(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"I/O tensors must be float32 or bfloat16, got {t.dtype}")


def _req(t, name, dtype=None, device=None):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def workspace_size(B, H, T, d_qk, d_v, chunk, io: int, variant: str = "auto") -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mlstm_fwd_chunkwise_workspace_size_variant(
        B, H, T, d_qk, d_v, chunk, io, VARIANTS[variant], ctypes.byref(n)))
    return n.value


def schedule(B, H, T, d_qk, d_v, chunk, io: int, variant: str = "auto"):
    """(kernel chunk length, segments per sequence) of a chunkwise call."""
    kc, ns = ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().mlstm_fwd_chunkwise_schedule(B, H, T, d_qk, d_v, chunk, io, VARIANTS[variant],
                                              ctypes.byref(kc), ctypes.byref(ns)))
    return kc.value, ns.value


def fwd_chunkwise(q, k, v, i_pre, f_pre, o_pre, C0=None, n0=None, m0=None, *, chunk: int = 64,
                  return_state: bool = True, variant: str = "auto", h=None, C_T=None, n_T=None,
                  m_T=None, workspace=None):
    """Chunkwise forward over whole sequences.

    q, k [B,H,T,d_qk], v, o_pre [B,H,T,d_v] (float32 or bfloat16, one dtype);
    i_pre, f_pre [B,H,T] float32; optional (C0 [B,H,d_qk,d_v], n0 [B,H,d_qk],
    m0 [B,H]) float32.  Returns h, or (h, (C_T, n_T, m_T)) with
    ``return_state``.  Output buffers may be passed in (C_T may be C0 for an
    in-place state update)."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io_t = q.dtype
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("o_pre", o_pre)):
        _req(t, name, io_t, dev)
    for name, t in (("i_pre", i_pre), ("f_pre", f_pre), ("C0", C0), ("n0", n0), ("m0", m0)):
        _req(t, name, torch.float32, dev)
    if h is None:
        h = torch.empty((B, H, T, dv), dtype=io_t, device=dev)
    if return_state and C_T is None:
        C_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
        n_T = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
        m_T = torch.empty((B, H), dtype=torch.float32, device=dev)
    io = _io(q)
    nbytes = workspace_size(B, H, T, dk, dv, chunk, io, variant)
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mlstm_fwd_chunkwise_variant(
        _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre),
        _ptr(C0), _ptr(n0), _ptr(m0), _ptr(h), _ptr(C_T), _ptr(n_T), _ptr(m_T),
        B, H, T, dk, dv, chunk, io, VARIANTS[variant],
        _ptr(workspace), ws_len, _stream(dev)))
    if return_state:
        return h, (C_T, n_T, m_T)
    return h


def bwd_workspace_size(B, H, T, d_qk, d_v, chunk, io: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mlstm_bwd_chunkwise_workspace_size(B, H, T, d_qk, d_v, chunk, io, ctypes.byref(n)))
    return n.value


def bwd_chunkwise(q, k, v, i_pre, f_pre, o_pre, dh, C0=None, n0=None, m0=None, *, chunk: int = 32,
                  state_grad: bool = False, workspace=None):
    """Gradients of a loss L given dL/dh, for the inputs of fwd_chunkwise.

    Same inputs as fwd_chunkwise plus dh [B,H,T,d_v] (the I/O dtype).
    Returns float32 (dq, dk, dv, di, df, do), and with ``state_grad`` also
    (dC0, dn0, dm0) -- of the zero state when no initial state is given."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io_t = q.dtype
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("o_pre", o_pre), ("dh", dh)):
        _req(t, name, io_t, dev)
    for name, t in (("i_pre", i_pre), ("f_pre", f_pre), ("C0", C0), ("n0", n0), ("m0", m0)):
        _req(t, name, torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    gq, gk = torch.empty((B, H, T, dk), **f32), torch.empty((B, H, T, dk), **f32)
    gv, go = torch.empty((B, H, T, dv), **f32), torch.empty((B, H, T, dv), **f32)
    gi, gf = torch.empty((B, H, T), **f32), torch.empty((B, H, T), **f32)
    gC0 = gn0 = gm0 = None
    if state_grad:
        gC0, gn0, gm0 = (torch.empty((B, H, dk, dv), **f32), torch.empty((B, H, dk), **f32),
                         torch.empty((B, H), **f32))
    io = _io(q)
    nbytes = bwd_workspace_size(B, H, T, dk, dv, chunk, io)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    _check(lib().mlstm_bwd_chunkwise(
        _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre),
        _ptr(C0), _ptr(n0), _ptr(m0), _ptr(dh), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(gi), _ptr(gf),
        _ptr(go), _ptr(gC0), _ptr(gn0), _ptr(gm0), B, H, T, dk, dv, chunk, io,
        _ptr(workspace), ws_len, _stream(dev)))
    out = (gq, gk, gv, gi, gf, go)
    if state_grad:
        return out + (gC0, gn0, gm0)
    return out


def layer_workspace_size(B, T, d_model, H, d_qk, d_v, chunk, io: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mlstm_layer_fwd_workspace_size(B, T, d_model, H, d_qk, d_v, chunk, io, ctypes.byref(n)))
    return n.value


def layer_fwd(x, W_q, W_k, W_v, W_o, W_i, W_f, b_q, b_k, b_v, b_o, b_i, b_f, C0=None, n0=None,
              m0=None, *, chunk: int = 64, return_state: bool = True, workspace=None):
    """The mLSTM layer forward (input projections, then the chunkwise cell).

    x [B,T,d_model]; W_q, W_k [H,d_qk,d_model]; W_v, W_o [H,d_v,d_model];
    W_i, W_f [H,d_model] (all the I/O dtype); biases float32 b_q, b_k [H,d_qk],
    b_v, b_o [H,d_v], b_i, b_f [H]; optional state C0 [H,B,d_qk,d_v], n0
    [H,B,d_qk], m0 [H,B].  Cells are head-major.  Returns h [H,B,T,d_v], or
    (h, (C_T, n_T, m_T)) with ``return_state``."""
    import torch
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io_t = x.dtype
    B, T, D = x.shape
    H, dk = W_q.shape[0], W_q.shape[1]
    dv = W_v.shape[1]
    for name, t in (("x", x), ("W_q", W_q), ("W_k", W_k), ("W_v", W_v), ("W_o", W_o), ("W_i", W_i),
                    ("W_f", W_f)):
        _req(t, name, io_t, dev)
    for name, t in (("b_q", b_q), ("b_k", b_k), ("b_v", b_v), ("b_o", b_o), ("b_i", b_i), ("b_f", b_f),
                    ("C0", C0), ("n0", n0), ("m0", m0)):
        _req(t, name, torch.float32, dev)
    h = torch.empty((H, B, T, dv), dtype=io_t, device=dev)
    C_T = n_T = m_T = None
    if return_state:
        f32 = dict(dtype=torch.float32, device=dev)
        C_T, n_T, m_T = (torch.empty((H, B, dk, dv), **f32), torch.empty((H, B, dk), **f32),
                         torch.empty((H, B), **f32))
    io = _io(x)
    if workspace is None:
        workspace = torch.empty(layer_workspace_size(B, T, D, H, dk, dv, chunk, io), dtype=torch.uint8,
                                device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    _check(lib().mlstm_layer_fwd(
        _ptr(x), _ptr(W_q), _ptr(W_k), _ptr(W_v), _ptr(W_o), _ptr(W_i), _ptr(W_f),
        _ptr(b_q), _ptr(b_k), _ptr(b_v), _ptr(b_o), _ptr(b_i), _ptr(b_f),
        _ptr(C0), _ptr(n0), _ptr(m0), _ptr(h), _ptr(C_T), _ptr(n_T), _ptr(m_T),
        B, T, D, H, dk, dv, chunk, io, _ptr(workspace), ws_len, _stream(dev)))
    return (h, (C_T, n_T, m_T)) if return_state else h


def slstm_fwd(gx, R, c0=None, n0=None, m0=None, h0=None, *, return_state: bool = True, h=None,
              c_T=None, n_T=None, m_T=None, h_T=None):
    """The sLSTM cell forward.

    gx [B,H,T,4,d] (input part of the z, i, f, o pre-activations) and R
    [H,4,d,d] (recurrent weights) in the I/O dtype; optional state c0, n0,
    m0, h0 [B,H,d] float32.  Returns h [B,H,T,d], or (h, (c_T, n_T, m_T,
    h_T)) with ``return_state``."""
    import torch
    dev = gx.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io_t = gx.dtype
    B, H, T, four, d = gx.shape
    if four != 4:
        raise ValueError("gx must be [B, H, T, 4, d]")
    _req(gx, "gx", io_t, dev)
    _req(R, "R", io_t, dev)
    for name, t in (("c0", c0), ("n0", n0), ("m0", m0), ("h0", h0)):
        _req(t, name, torch.float32, dev)
    if h is None:
        h = torch.empty((B, H, T, d), dtype=io_t, device=dev)
    if return_state and c_T is None:
        f32 = dict(dtype=torch.float32, device=dev)
        c_T, n_T, m_T, h_T = (torch.empty((B, H, d), **f32) for _ in range(4))
    _check(lib().mlstm_slstm_fwd(
        _ptr(gx), _ptr(R), _ptr(c0), _ptr(n0), _ptr(m0), _ptr(h0), _ptr(h),
        _ptr(c_T), _ptr(n_T), _ptr(m_T), _ptr(h_T), B, H, T, d, _io(gx), _stream(dev)))
    return (h, (c_T, n_T, m_T, h_T)) if return_state else h


def step_workspace_size(B, H, d_qk, d_v, io: int) -> int:
    """Bytes of workspace mlstm_step can use for this shape (0: none)."""
    n = ctypes.c_size_t(0)
    _check(lib().mlstm_step_workspace_size(B, H, d_qk, d_v, io, ctypes.byref(n)))
    return n.value


def step_workspace(B, H, d_qk, d_v, io_dtype, device):
    """A workspace for mlstm_step (None when the shape uses none): scratch that
    any later calls on the same stream may reuse."""
    import torch
    n = step_workspace_size(B, H, d_qk, d_v, BF16 if io_dtype == torch.bfloat16 else F32)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def step(q, k, v, i_pre, f_pre, o_pre, C=None, n=None, m=None, *, h=None, C_out=None,
         n_out=None, m_out=None, inplace: bool = True, split: bool = True, workspace=None):
    """One recurrent step for B*H cells.

    q, k [B,H,d_qk], v, o_pre [B,H,d_v]; i_pre, f_pre [B,H]; state (C [B,H,d_qk,
    d_v], n [B,H,d_qk], m [B,H]) float32 or None for the zero state.  With
    ``inplace`` (default) and a state given, the state tensors are updated in
    place.  ``split`` runs the row-split kernel where the shape has one, with
    ``workspace`` (from step_workspace; a fresh one per call when None); ``split=False`` streams each cell with one workgroup.  Returns (h,
    C_out, n_out, m_out)."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io_t = q.dtype
    B, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("o_pre", o_pre)):
        _req(t, name, io_t, dev)
    for name, t in (("i_pre", i_pre), ("f_pre", f_pre), ("C", C), ("n", n), ("m", m)):
        _req(t, name, torch.float32, dev)
    if h is None:
        h = torch.empty((B, H, dv), dtype=io_t, device=dev)
    if C_out is None:
        if inplace and C is not None:
            C_out, n_out, m_out = C, n, m
        else:
            C_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
            n_out = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
            m_out = torch.empty((B, H), dtype=torch.float32, device=dev)
    if not split:
        workspace = None
    elif workspace is None:
        workspace = step_workspace(B, H, dk, dv, io_t, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mlstm_step(
        _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre),
        _ptr(C), _ptr(n), _ptr(m), _ptr(h), _ptr(C_out), _ptr(n_out), _ptr(m_out),
        B, H, dk, dv, _io(q), _ptr(workspace), ws_bytes, _stream(dev)))
    return h, C_out, n_out, m_out


def step_noalloc(q, k, v, i_pre, f_pre, o_pre, C=None, n=None, m=None, *, h=None, C_out=None,
                 n_out=None, m_out=None, inplace: bool = True):
    """``step`` through mlstm_step_noalloc: the row split's workspace is the
    library's fixed per-device scratch (nothing is allocated by the library;
    outputs not given are allocated here, by torch, before the call).  Same
    arguments and result as ``step`` with ``split=True``."""
    import torch
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    io_t = q.dtype
    B, H, dk = q.shape
    dv = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("o_pre", o_pre)):
        _req(t, name, io_t, dev)
    for name, t in (("i_pre", i_pre), ("f_pre", f_pre), ("C", C), ("n", n), ("m", m)):
        _req(t, name, torch.float32, dev)
    if h is None:
        h = torch.empty((B, H, dv), dtype=io_t, device=dev)
    if C_out is None:
        if inplace and C is not None:
            C_out, n_out, m_out = C, n, m
        else:
            C_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
            n_out = torch.empty((B, H, dk), dtype=torch.float32, device=dev)
            m_out = torch.empty((B, H), dtype=torch.float32, device=dev)
    _check(lib().mlstm_step_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre),
        _ptr(C), _ptr(n), _ptr(m), _ptr(h), _ptr(C_out), _ptr(n_out), _ptr(m_out),
        B, H, dk, dv, _io(q), _stream(dev)))
    return h, C_out, n_out, m_out
