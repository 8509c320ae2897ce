"""GPU parity of the mLSTM layer forward (mlstm_layer_fwd: hipBLASLt
projections + gate-bias kernel + chunkwise cell) against the float64 layer
oracle (oracle/layer.py) on seeded workloads.

Both sides take the same inputs (x and the weights already in the I/O dtype)
and both hand the cell q, k, v, o~ in the I/O dtype: the library rounds its
float32 GEMM results, the oracle its float64 projections.  The tolerances
are the cell's (2e-3 float32, 2e-2 bfloat16, per-row relative)."""
import numpy as np
import pytest
import torch

from oracle import layer as L
from tests import parity as PT
from xlstm_mlstm_matrix_amd import binding, inputs as I

pytestmark = pytest.mark.gpu

NAMES = ("x", "W_q", "W_k", "W_v", "W_o", "W_i", "W_f", "b_q", "b_k", "b_v", "b_o", "b_i", "b_f")


def run_gpu(d, chunk):
    g = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    h, (C, n, m) = binding.layer_fwd(*(g[k] for k in NAMES), g["C0"], g["n0"], g["m0"], chunk=chunk)
    torch.cuda.synchronize()
    return h, C, n, m


def run_oracle(d, io):
    return L.layer_forward(*(d[k] for k in NAMES), d["C0"], d["n0"], d["m0"], io=io)


def compare(gpu, ref, io, what):
    h, C, n, m = gpu
    H, B, T, dv = h.shape
    P = H * B
    flat = lambda t, r: (t.reshape(P, *t.shape[2:]), r.reshape(P, *r.shape[2:]))
    pairs = [flat(x, r) for x, r in zip((h, C, n, m), ref)]
    PT.compare_fwd(tuple(p[0] for p in pairs), tuple(p[1] for p in pairs), io, what)


def test_layer_small_f32():
    """B=2 T=100 d_model=64 H=2 d_qk=16 d_v=32, float32, random initial state."""
    w = I.layer_workload("layer_small")
    d = I.gen_layer(w)
    compare(run_gpu(d, w.chunk), run_oracle(d, "f32"), "f32", "layer small f32")


def test_layer_small_bf16_zero_state():
    w = I.layer_workload("layer_small", io="bf16", init_state=None)
    d = I.gen_layer(w)
    compare(run_gpu(d, w.chunk), run_oracle(d, "bf16"), "bf16", "layer small bf16")


@pytest.mark.parametrize("T", [1, 63, 200])
def test_layer_7b_heads_short(T):
    """The 7B layer's heads (d_qk 256, d_v 512, bf16, chunk 64: the timed
    cell kernel) with a reduced d_model and batch, ragged lengths."""
    w = I.layer_workload("layer_7b_bf16", B=2, T=T, d_model=512, H=2)
    d = I.gen_layer(w)
    compare(run_gpu(d, w.chunk), run_oracle(d, "bf16"), "bf16", f"layer 7b heads T={T}")


@pytest.mark.parametrize("H,B,T", [(1, 1, 77), (3, 1, 33)])
def test_layer_7b_heads_odd_token_count(H, B, T):
    """The 7B layer's heads with H*B*T not a multiple of 4: the projections
    still run over all heads, but the gate pre-activations take two GEMMs
    (one [B*T, 2H] GEMM would leave f~ misaligned behind i~); with a random
    initial state."""
    w = I.layer_workload("layer_7b_bf16", B=B, T=T, d_model=256, H=H,
                         init_state={"C0": ("normal", 0.0, 0.1), "n0": ("normal", 0.0, 0.1),
                                     "m0": ("uniform", -1.0, 1.0)})
    d = I.gen_layer(w)
    compare(run_gpu(d, w.chunk), run_oracle(d, "bf16"), "bf16", f"layer 7b heads H={H} B={B} T={T}")


def test_layer_full_size_sampled():
    """The 7B layer workload at full size (B=8 T=4096 d_model=4096 H=8, the
    configuration the benchmark times); the oracle follows every head of two
    sampled batch rows."""
    w = I.layer_workload("layer_7b_bf16")
    print("[case] layer full size: generating inputs", flush=True)
    d = I.gen_layer(w, threads=16)
    h, C, n, m = run_gpu(d, w.chunk)
    print("[case] layer full size: GPU done", flush=True)
    for b in (1, 6):
        db = dict(d)
        db["x"] = d["x"][b:b + 1]
        ref = run_oracle(db, "bf16")
        compare((h[:, b:b + 1], C[:, b:b + 1], n[:, b:b + 1], m[:, b:b + 1]), ref, "bf16",
                f"layer full size, batch row {b}")


def test_layer_state_roundtrip_equals_one_call():
    """Two calls over halves of the sequence, the second seeded with the
    first's final state, equal one call over the whole sequence."""
    w = I.layer_workload("layer_small", T=96, init_state=None)
    d = I.gen_layer(w)
    h_all, C_all, n_all, m_all = run_gpu(d, w.chunk)
    d1 = dict(d); d1["x"] = d["x"][:, :40].contiguous()
    h1, C1, n1, m1 = run_gpu(d1, w.chunk)
    d2 = dict(d); d2["x"] = d["x"][:, 40:].contiguous()
    d2["C0"], d2["n0"], d2["m0"] = C1.cpu(), n1.cpu(), m1.cpu()
    h2, C2, n2, m2 = run_gpu(d2, w.chunk)
    h = torch.cat([h1, h2], dim=2)
    ref = run_oracle(d, "f32")
    compare((h, C2, n2, m2), ref, "f32", "layer in two calls")
    assert PT.row_relerr(PT.to_np(h), PT.to_np(h_all)) <= 1e-4


def test_layer_unsupported_d_model_raises():
    w = I.layer_workload("layer_small", d_model=60)
    d = I.gen_layer(w)
    with pytest.raises(binding.MlstmError):
        run_gpu(d, w.chunk)
