"""GPU parity of the sLSTM cell forward (mlstm_slstm_fwd) against the
float64 sLSTM oracle (oracle/slstm_ref.c) on seeded workloads.

Both sides take the same inputs (gx and R already in the I/O dtype).  h is
compared per token (one d-vector per row, max |x - r| / max |r|), the final
c and n after rescaling by e^{m_gpu - m_ref} (both are kept stabilized), m by
absolute error, h_T like h; tolerances 2e-3 (float32) and 2e-2 (bfloat16)."""
import numpy as np
import pytest
import torch

from oracle import slstm as S
from tests import parity as PT
from xlstm_mlstm_matrix_amd import binding, inputs as I

pytestmark = pytest.mark.gpu


def run_gpu(d, **kw):
    g = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    h, st = binding.slstm_fwd(g["gx"], g["R"], g["c0"], g["n0"], g["m0"], g["h0"], **kw)
    torch.cuda.synchronize()
    return h, st


def run_oracle(d, groups=None):
    R = d["R"]
    if groups is not None:                       # [1, P] groups with their own heads
        R = R[[h for _, h in groups]]
        gx = d["gx"].reshape(1, len(groups), *d["gx"].shape[2:])
        hs, sts = [], []
        for p in range(len(groups)):
            h, st = S.forward(gx[:, p:p + 1], R[p:p + 1],
                              *((None,) * 4 if d["c0"] is None else (d[k][:, p:p + 1] for k in ("c0", "n0", "m0", "h0"))))
            hs.append(h); sts.append(st)
        return np.concatenate(hs, axis=1), tuple(np.concatenate([s[i] for s in sts], axis=1) for i in range(4))
    st = (None,) * 4 if d["c0"] is None else tuple(d[k] for k in ("c0", "n0", "m0", "h0"))
    return S.forward(d["gx"], R, *st)


def compare(gpu, ref, io, what):
    (h, (c, n, m, hT)), (hr, (cr, nr, mr, hTr)) = gpu, ref
    h, c, n, m, hT = (PT.to_np(x) for x in (h, c, n, m, hT))
    d = h.shape[-1]
    assert np.all(np.isfinite(h)), what
    eh = PT.row_relerr(h.reshape(-1, d), hr.reshape(-1, d))
    sc = np.exp(m - mr)
    ec = PT.row_relerr((c * sc).reshape(-1, d), cr.reshape(-1, d))
    en = PT.row_relerr((n * sc).reshape(-1, d), nr.reshape(-1, d))
    em = float(np.max(np.abs(m - mr)))
    ehT = PT.row_relerr(hT.reshape(-1, d), hTr.reshape(-1, d))
    print(f"[parity] {what}: h {eh:.2e}  c {ec:.2e}  n {en:.2e}  m {em:.2e}  h_T {ehT:.2e}", flush=True)
    tol = PT.TOL[io]
    assert eh <= tol and ec <= tol and en <= tol and ehT <= tol, what
    assert em <= PT.TOL_M[io], what


def test_small_f32_with_state():
    w = I.slstm_workload("slstm_small")
    d = I.gen_slstm(w)
    compare(run_gpu(d), run_oracle(d), "f32", "slstm small f32")


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dd", [16, 48, 64, 112, 128])
def test_head_dims(io, dd):
    w = I.slstm_workload("slstm_small", d=dd, io=io, T=67, state=(io == "f32"))
    d = I.gen_slstm(w)
    compare(run_gpu(d), run_oracle(d), io, f"slstm d={dd} {io}")


@pytest.mark.parametrize("T", [1, 7, 8, 9])
def test_lengths_around_the_prefetch_ring(T):
    """T below, at and just past the 8 steps of input held in flight."""
    w = I.slstm_workload("slstm_small", T=T)
    d = I.gen_slstm(w)
    compare(run_gpu(d), run_oracle(d), "f32", f"slstm T={T}")


def test_state_carry_and_in_place():
    """Two calls chained through the state (the second one updating the state
    tensors in place) equal one call."""
    w = I.slstm_workload("slstm_small", T=90)
    d = I.gen_slstm(w)
    h_all, st_all = run_gpu(d)
    g = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    st = [g[k].clone() for k in ("c0", "n0", "m0", "h0")]
    h1 = binding.slstm_fwd(g["gx"][:, :, :40].contiguous(), g["R"], *st, return_state=False)
    # the first call's final state, written over its own initial state
    binding.slstm_fwd(g["gx"][:, :, :40].contiguous(), g["R"], *st, c_T=st[0], n_T=st[1], m_T=st[2],
                      h_T=st[3])
    h2, st2 = binding.slstm_fwd(g["gx"][:, :, 40:].contiguous(), g["R"], *st)
    torch.cuda.synchronize()
    h = torch.cat([h1, h2], dim=2)
    assert PT.row_relerr(PT.to_np(h).reshape(-1, w.d), PT.to_np(h_all).reshape(-1, w.d)) <= 1e-5
    compare((h, st2), run_oracle(d), "f32", "slstm in two calls")


def test_full_size_sampled():
    """The benchmark's workload (B=16 H=8 T=4096 d=128, bf16) at full size;
    the oracle follows four sampled groups."""
    w = I.slstm_workload("slstm_bf16")
    print("[case] slstm full size: generating inputs", flush=True)
    d = I.gen_slstm(w, threads=16)
    h, st = run_gpu(d)
    print("[case] slstm full size: GPU done", flush=True)
    groups = [(0, 0), (5, 3), (11, 6), (15, 7)]
    ds = I.gen_slstm(w, groups=groups)
    hr, str_ = run_oracle(ds, groups=groups)
    sel = lambda x: torch.stack([x[b, hh] for b, hh in groups]).unsqueeze(0)
    compare((sel(h), tuple(sel(x) for x in st)), (hr, str_), "bf16", "slstm full size, 4 groups")


def test_unsupported_head_dim_raises():
    w = I.slstm_workload("slstm_small", d=144, T=5)
    d = I.gen_slstm(w)
    with pytest.raises(binding.MlstmError):
        run_gpu(d)
