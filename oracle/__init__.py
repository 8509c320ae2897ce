"""Float64 CPU oracle of the mLSTM cell forward and backward passes (test
infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It wraps ``mlstm_ref.c`` (the plain sequential
recurrence in float64, see that file's header for the equations and their
sources) through ctypes, and shares no code with the HIP library.  The
submodule ``oracle.layer`` adds the layer's input projections (float64
matrix products) in front of that recurrence; ``oracle.slstm`` wraps
``slstm_ref.c``, the float64 sLSTM cell.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mlstm_ref.c")
LIB = os.path.join(HERE, "libmlstm_ref.so")

__all__ = ["build", "load", "forward", "backward", "Oracle", "SRC", "LIB"]


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O3, IEEE semantics kept: no fast-math, so
    floating-point sums keep their written order)."""
    cmd = ["gcc", "-std=c99", "-O3", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror",
           *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path} (run oracle.build())")
        self.lib = ctypes.CDLL(path)
        f = self.lib.mlstm_ref_forward
        dp = ctypes.POINTER(ctypes.c_double)
        f.argtypes = [dp] * 13 + [ctypes.c_long] * 4 + [ctypes.c_int]
        f.restype = ctypes.c_int
        self._f = f
        b = self.lib.mlstm_ref_backward
        b.argtypes = [dp] * 19 + [ctypes.c_long] * 4 + [ctypes.c_int]
        b.restype = ctypes.c_int
        self._b = b

    def forward(self, q, k, v, i_pre, f_pre, o_pre, C0=None, n0=None, m0=None,
                threads: int = 0):
        """Run the recurrence over P pairs.

        q, k: [P, T, d_qk]; v, o_pre: [P, T, d_v]; i_pre, f_pre: [P, T];
        optional initial state C0 [P, d_qk, d_v], n0 [P, d_qk], m0 [P].
        Inputs may be numpy arrays or torch tensors of any float dtype; each is
        converted exactly to float64.  Returns (h, C_T, n_T, m_T) as float64
        numpy arrays."""
        q, k, v, i_pre, f_pre, o_pre = (_f64(x) for x in (q, k, v, i_pre, f_pre, o_pre))
        P, T, dk = q.shape
        dv = v.shape[2]
        assert k.shape == (P, T, dk) and v.shape == (P, T, dv) and o_pre.shape == (P, T, dv)
        assert i_pre.shape == (P, T) and f_pre.shape == (P, T)
        have = [x is not None for x in (C0, n0, m0)]
        if any(have) and not all(have):
            raise ValueError("initial state must be given completely or not at all")
        if all(have):
            C0, n0, m0 = _f64(C0), _f64(n0), _f64(m0)
            assert C0.shape == (P, dk, dv) and n0.shape == (P, dk) and m0.shape == (P,)
        h = np.empty((P, T, dv))
        C = np.empty((P, dk, dv))
        n = np.empty((P, dk))
        m = np.empty((P,))
        rc = self._f(_p(q), _p(k), _p(v), _p(i_pre), _p(f_pre), _p(o_pre),
                     _p(C0), _p(n0), _p(m0), _p(h), _p(C), _p(n), _p(m),
                     P, T, dk, dv, int(threads))
        if rc != 0:
            raise RuntimeError(f"mlstm_ref_forward failed with code {rc}")
        return h, C, n, m

    def backward(self, q, k, v, i_pre, f_pre, o_pre, dh, C0=None, n0=None, m0=None,
                 threads: int = 0):
        """Gradients of sum(dh * h) (dh: [P, T, d_v]) with respect to every
        input and the initial state: returns (dq, dk, dv, di, df, do, dC0,
        dn0, dm0) as float64 numpy arrays (the initial-state gradients are
        those of the zero state when none is given)."""
        q, k, v, i_pre, f_pre, o_pre, dh = (_f64(x) for x in (q, k, v, i_pre, f_pre, o_pre, dh))
        P, T, dk = q.shape
        dv = v.shape[2]
        assert k.shape == (P, T, dk) and v.shape == (P, T, dv) and o_pre.shape == (P, T, dv)
        assert i_pre.shape == (P, T) and f_pre.shape == (P, T) and dh.shape == (P, T, dv)
        have = [x is not None for x in (C0, n0, m0)]
        if any(have) and not all(have):
            raise ValueError("initial state must be given completely or not at all")
        if all(have):
            C0, n0, m0 = _f64(C0), _f64(n0), _f64(m0)
            assert C0.shape == (P, dk, dv) and n0.shape == (P, dk) and m0.shape == (P,)
        out = [np.empty((P, T, dk)), np.empty((P, T, dk)), np.empty((P, T, dv)), np.empty((P, T)),
               np.empty((P, T)), np.empty((P, T, dv)), np.empty((P, dk, dv)), np.empty((P, dk)),
               np.empty((P,))]
        rc = self._b(_p(q), _p(k), _p(v), _p(i_pre), _p(f_pre), _p(o_pre), _p(C0), _p(n0), _p(m0), _p(dh),
                     *(_p(x) for x in out), P, T, dk, dv, int(threads))
        if rc != 0:
            raise RuntimeError(f"mlstm_ref_backward failed with code {rc}")
        return tuple(out)


def _f64(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


_DEFAULT: Optional[Oracle] = None


def load() -> Oracle:
    """The oracle built in-tree (built on first use if missing)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _DEFAULT = Oracle(LIB)
    return _DEFAULT


def forward(*args, **kw):
    """``load().forward(...)``."""
    return load().forward(*args, **kw)


def backward(*args, **kw):
    """``load().backward(...)``."""
    return load().backward(*args, **kw)
