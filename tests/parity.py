"""Helpers of the GPU parity tests: run the HIP path and the float64 oracle on
the same seeded inputs and compare.

Error metric (the tolerance is a maximum relative error; the pages give no
formula for it): per output row -- one token's h vector, one pair's C or n --
max_j |x_j - r_j| / max_j |r_j|, maximised over rows.  Final states are
compared in the oracle's stabilizer: C_gpu * e^{m_gpu - m_ref} against C_ref;
m itself (a log value) by absolute error.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from xlstm_mlstm_matrix_amd import binding, inputs

TOL = {"f32": 2e-3, "bf16": 2e-2}
TOL_M = {"f32": 1e-4, "bf16": 1e-3}


def row_relerr(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if x.size == 0:
        return 0.0
    num = np.abs(x - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    return float(np.max(num / np.maximum(den, 1e-30)))


def to_np(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def cuda(d):
    return {k: (v.cuda() if v is not None else None) for k, v in d.items()}


def run_gpu_fwd(d, chunk, variant="auto", io=None):
    """d: dict from inputs.gen_prefill ([P, T, ...]); runs as B=1, H=P."""
    g = cuda(d)
    P, T, dk = g["q"].shape
    add = lambda t: None if t is None else t.unsqueeze(0)
    h, (C, n, m) = binding.fwd_chunkwise(
        add(g["q"]), add(g["k"]), add(g["v"]), add(g["i_pre"]), add(g["f_pre"]), add(g["o_pre"]),
        add(g["C0"]), add(g["n0"]), add(g["m0"]), chunk=chunk, variant=variant)
    torch.cuda.synchronize()
    return h[0], C[0], n[0], m[0]


def run_oracle(d, threads=0):
    st = (d["C0"], d["n0"], d["m0"]) if d["C0"] is not None else (None, None, None)
    return oracle.forward(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"], *st,
                          threads=threads)


def compare_fwd(gpu, ref, io, what=""):
    h, C, n, m = (to_np(x) for x in gpu)
    hr, Cr, nr, mr = ref
    assert np.all(np.isfinite(h)), f"{what}: non-finite h"
    eh = row_relerr(h, hr)
    scale = np.exp(m - mr)
    eC = row_relerr((C * scale[:, None, None]).reshape(C.shape[0], -1), Cr.reshape(Cr.shape[0], -1))
    en = row_relerr(n * scale[:, None], nr)
    em = float(np.max(np.abs(m - mr)))
    print(f"[parity] {what}: h {eh:.2e}  C {eC:.2e}  n {en:.2e}  m {em:.2e}", flush=True)
    assert eh <= TOL[io], (what, "h", eh)
    assert eC <= TOL[io], (what, "C", eC)
    assert en <= TOL[io], (what, "n", en)
    assert em <= TOL_M[io], (what, "m", em)
    return eh, eC, en, em


def m_closed_form(i_pre, f_pre, m0=None):
    """Stabilizer after the whole sequence, from the gates alone:
    max(m0 + sum f~, max_s (i~_s + sum_{r>s} f~_r)); float64, any leading shape."""
    i = np.asarray(i_pre, dtype=np.float64)
    f = np.asarray(f_pre, dtype=np.float64)
    tail = np.cumsum(f[..., ::-1], axis=-1)[..., ::-1]  # sum_{r>=s}
    tail = tail - f                                     # sum_{r>s}
    base = (0.0 if m0 is None else np.asarray(m0, dtype=np.float64)) + f.sum(axis=-1)
    return np.maximum(base, np.max(i + tail, axis=-1))
