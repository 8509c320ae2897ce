"""Float64 oracle of the mLSTM layer forward: the input projections feeding
the cell (test infrastructure; only the tests, ``__graft_entry__.smoke()``
and the benchmark's CPU-baseline leg may import it).

Follows the example mLSTM module on the xLSTM notes page (section "mLSTM",
its listing of the recurrent forward): from a token x_t of width d_model,
linear maps with bias give the query, key and value, a scalar input-gate and
forget-gate pre-activation, and the output-gate pre-activation; the forget
pre-activation enters the stabilized recurrence as the log of the forget
gate and the output gate is its sigmoid.  Readings (the page shows a single
head):

- with H heads each head has its own projections: W_q[h], W_k[h] of shape
  [d_qk, d_model], W_v[h], W_o[h] of shape [d_v, d_model], W_i[h], W_f[h] of
  shape [d_model], and biases of the matching widths;
- the (batch, head) cells are ordered head-major: cell p = h*B + b, so every
  per-cell tensor is [H, B, ...];
- the cell is the oracle's sequential recurrence (``oracle.forward``) from the
  given state or the zero state;
- with bfloat16 I/O the cell's inputs q, k, v and o~ are bfloat16 tensors,
  so the float64 projections are rounded to bfloat16 (to nearest, ties to
  even, straight from float64) before the cell; the gate pre-activations stay
  float64.

Each projection is a float64 matrix product (a library primitive), nothing
fused or reordered.
"""
from __future__ import annotations

import numpy as np

from . import forward as cell_forward

__all__ = ["layer_forward", "projections", "round_bf16"]


def round_bf16(a):
    """float64 -> the nearest bfloat16 value (8 significant bits, ties to
    even), returned as float64; normal range only (no overflow or subnormal
    handling, none occur here)."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                         # a = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def projections(x, W_q, W_k, W_v, W_o, W_i, W_f, b_q, b_k, b_v, b_o, b_i, b_f):
    """The listing's linear maps for every head: returns q, k [H, B, T, d_qk],
    v, o_pre [H, B, T, d_v] and i_pre, f_pre [H, B, T] in float64."""
    x = _f64(x)                                   # [B, T, D]
    out = []
    for W, b in ((W_q, b_q), (W_k, b_k), (W_v, b_v), (W_o, b_o)):
        W, b = _f64(W), _f64(b)                   # [H, d, D], [H, d]
        y = np.stack([x @ W[h].T + b[h] for h in range(W.shape[0])])   # [H, B, T, d]
        out.append(y)
    for W, b in ((W_i, b_i), (W_f, b_f)):
        W, b = _f64(W), _f64(b)                   # [H, D], [H]
        out.append(np.stack([x @ W[h] + b[h] for h in range(W.shape[0])]))  # [H, B, T]
    return tuple(out)


def layer_forward(x, W_q, W_k, W_v, W_o, W_i, W_f, b_q, b_k, b_v, b_o, b_i, b_f,
                  C0=None, n0=None, m0=None, io: str = "f32", threads: int = 0):
    """x [B, T, d_model]; weights and biases as in ``projections``; optional
    state C0 [H, B, d_qk, d_v], n0 [H, B, d_qk], m0 [H, B]; io "f32" or
    "bf16" (the cell's I/O dtype).  Returns h [H, B, T, d_v] and the final
    state (C [H, B, d_qk, d_v], n [H, B, d_qk], m [H, B]), float64."""
    q, k, v, o, i, f = projections(x, W_q, W_k, W_v, W_o, W_i, W_f, b_q, b_k, b_v, b_o, b_i, b_f)
    if io == "bf16":
        q, k, v, o = (round_bf16(a) for a in (q, k, v, o))
    elif io != "f32":
        raise ValueError(f"unknown io dtype {io!r}")
    H, B, T, dk = q.shape
    dv = v.shape[-1]
    P = H * B
    st = (None, None, None)
    if C0 is not None:
        st = (_f64(C0).reshape(P, dk, dv), _f64(n0).reshape(P, dk), _f64(m0).reshape(P))
    h, C, n, m = cell_forward(q.reshape(P, T, dk), k.reshape(P, T, dk), v.reshape(P, T, dv),
                              i.reshape(P, T), f.reshape(P, T), o.reshape(P, T, dv), *st,
                              threads=threads)
    return (h.reshape(H, B, T, dv), C.reshape(H, B, dk, dv), n.reshape(H, B, dk), m.reshape(H, B))
