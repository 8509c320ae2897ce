"""Float64 oracle of the sLSTM cell forward (test infrastructure; only the
tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import it).

Wraps ``slstm_ref.c`` (see its header for the recurrence and the readings
taken where the pages are silent) through ctypes.  Shares no code with the
HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "slstm_ref.c")
LIB = os.path.join(HERE, "libslstm_ref.so")

__all__ = ["build", "load", "forward", "SRC", "LIB"]


def build(src: str = SRC, out: str = LIB) -> str:
    cmd = ["gcc", "-std=c99", "-O3", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Werror", src, "-o", out,
           "-lm"]
    subprocess.run(cmd, check=True)
    return out


class SlstmOracle:
    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"sLSTM oracle library not built: {path}")
        self.lib = ctypes.CDLL(path)
        f = self.lib.slstm_ref_forward
        dp = ctypes.POINTER(ctypes.c_double)
        f.argtypes = [dp] * 11 + [ctypes.c_long] * 3 + [ctypes.c_int]
        f.restype = ctypes.c_int
        self._f = f

    def forward(self, gx, R, c0=None, n0=None, m0=None, h0=None, threads: int = 0):
        """gx [B, H, T, 4, d] (gate order z, i, f, o; the input part of each
        pre-activation); R [H, 4, d, d] (row j of R[h, g] feeds cell j);
        optional state c0, n0, m0, h0 [B, H, d].  Returns h [B, H, T, d] and
        the final state (c, n, m, h) [B, H, d] each, float64."""
        gx = _f64(gx)
        R = _f64(R)
        B, H, T, four, d = gx.shape
        assert four == 4 and R.shape == (H, 4, d, d)
        P = B * H
        Rp = np.ascontiguousarray(np.broadcast_to(R[None], (B, H, 4, d, d)).reshape(P, 4, d, d))
        have = [x is not None for x in (c0, n0, m0, h0)]
        if any(have) and not all(have):
            raise ValueError("initial state must be given completely or not at all")
        st = [None] * 4
        if all(have):
            st = [np.ascontiguousarray(_f64(x).reshape(P, d)) for x in (c0, n0, m0, h0)]
        h = np.empty((P, T, d))
        out = [np.empty((P, d)) for _ in range(4)]
        rc = self._f(_p(np.ascontiguousarray(gx.reshape(P, T, 4, d))), _p(Rp), *(_p(x) for x in st),
                     _p(h), *(_p(x) for x in out), P, T, d, int(threads))
        if rc != 0:
            raise RuntimeError(f"slstm_ref_forward failed with code {rc}")
        return h.reshape(B, H, T, d), tuple(x.reshape(B, H, d) for x in out)


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


_DEFAULT: Optional[SlstmOracle] = None


def load() -> SlstmOracle:
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _DEFAULT = SlstmOracle(LIB)
    return _DEFAULT


def forward(*args, **kw):
    return load().forward(*args, **kw)
