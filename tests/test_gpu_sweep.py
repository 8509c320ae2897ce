"""Seeded random-shape parity sweep of the forward, the recurrent step, the
backward, the layer forward and the sLSTM against the float64 oracles.

The fixed cases elsewhere pick their shapes by hand (tile edges, the
workloads' own sizes).  Here the head sizes, sequence length, chunk, I/O
dtype, schedule and initial state are drawn together from one seeded
generator, so that combinations nobody wrote down get run too: d_qk and d_v
any multiples of 16 up to 256 and 512, T from 1 to a few hundred, chunk 16 to
128, one to five (batch, head) pairs.  Inputs follow the workloads'
distributions (the small float32 workload for float32 I/O, the 7B-layer one
for bfloat16); the tolerances and the error metric are those of
tests/parity.py.  Every case prints its draw before it runs."""
import numpy as np
import pytest
import torch

from tests import parity as PT
from tests.test_gpu_backward import compare as bwd_compare, run_gpu as bwd_gpu, run_oracle as bwd_oracle
from tests.test_gpu_step import compare_steps, oracle_steps, run_steps
from tests.test_gpu_layer import compare as layer_compare, run_gpu as layer_gpu, run_oracle as layer_oracle
from tests.test_gpu_slstm import compare as slstm_compare, run_gpu as slstm_gpu, run_oracle as slstm_oracle
from xlstm_mlstm_matrix_amd import inputs as I

pytestmark = pytest.mark.gpu

N_FWD, N_STEP, N_BWD, N_LAYER, N_SLSTM = 48, 16, 12, 12, 12
# draws kept from a wider run, each of which once failed: 183 (float32, d_qk
# 176, chunk 32: the first token's q.k cancels ~7500-fold, beyond what
# operands of ~16 bits resolve to 2e-3)
EXTRA_FWD = [183]


def _draw(seed):
    return np.random.default_rng(seed)


def _pairs(rng, w, n):
    idx = rng.choice(w.B * w.H, size=n, replace=False)
    return [(int(i) // w.H, int(i) % w.H) for i in sorted(idx)]


def _random_state(rng, P, dk, dv):
    return (torch.from_numpy(rng.normal(0.0, 0.05, (P, dk, dv))).float(),
            torch.from_numpy(rng.normal(0.0, 0.05, (P, dk))).float(),
            torch.from_numpy(rng.uniform(-1.0, 1.0, P)).float())


def fwd_case(i):
    rng = _draw(7100 + i)
    io = ("f32", "bf16")[int(rng.integers(2))]
    dk = 16 * int(rng.integers(1, 17))
    dv = 16 * int(rng.integers(1, 33))
    T = int(rng.integers(1, 601))
    chunk = int(rng.choice([16, 32, 64, 128]))
    variant = ("auto", "fused", "segscan")[int(rng.integers(3))]
    P = int(rng.integers(1, 6))
    state = bool(rng.integers(2))
    return rng, dict(io=io, dk=dk, dv=dv, T=T, chunk=chunk, variant=variant, P=P, state=state)


@pytest.mark.parametrize("i", list(range(N_FWD)) + EXTRA_FWD)
def test_fwd_sweep(i):
    rng, c = fwd_case(i)
    print(f"[case] fwd sweep {i}: {c}", flush=True)
    name = "small_f32" if c["io"] == "f32" else "prefill_7b_bf16"
    w = I.workload(name, d_qk=c["dk"], d_v=c["dv"])
    d = I.gen_prefill(w, pairs=_pairs(rng, w, c["P"]), T=c["T"])
    if c["state"]:
        d["C0"], d["n0"], d["m0"] = _random_state(rng, c["P"], c["dk"], c["dv"])
    else:
        d["C0"] = d["n0"] = d["m0"] = None
    PT.compare_fwd(PT.run_gpu_fwd(d, c["chunk"], variant=c["variant"]), PT.run_oracle(d), c["io"],
                   f"fwd sweep {i}")


@pytest.mark.parametrize("i", range(N_STEP))
def test_step_sweep(i):
    rng = _draw(7300 + i)
    io = ("f32", "bf16")[int(rng.integers(2))]
    dk = 16 * int(rng.integers(1, 17))
    dv = 16 * int(rng.integers(1, 33))
    B = int(rng.integers(1, 5))
    S = int(rng.integers(1, 9))
    split = bool(rng.integers(2))
    state = bool(rng.integers(2))
    print(f"[case] step sweep {i}: io={io} dk={dk} dv={dv} B={B} steps={S} split={split} state={state}",
          flush=True)
    w = I.workload("decode_bf16", io=io, d_qk=dk, d_v=dv)
    steps = PT.cuda(I.gen_decode_steps(w, range(S), B=B))
    st = tuple(x.cuda() for x in I.gen_decode_state(w, B=B)) if state else None
    compare_steps(run_steps(steps, st, split=split), oracle_steps(steps, st), io, f"step sweep {i}")


@pytest.mark.parametrize("i", range(N_BWD))
def test_bwd_sweep(i):
    rng = _draw(7500 + i)
    io = ("f32", "bf16")[int(rng.integers(2))]
    dk = 16 * int(rng.integers(1, 17))
    dv = 16 * int(rng.integers(1, 33))
    # the oracle keeps every state of the sequence: T * d_qk * d_v doubles per pair
    T = int(rng.integers(1, max(2, min(301, 12_000_000 // (dk * dv)))))
    P = int(rng.integers(1, 4))
    state = bool(rng.integers(2))
    print(f"[case] bwd sweep {i}: io={io} dk={dk} dv={dv} T={T} P={P} state={state}", flush=True)
    name = "small_f32" if io == "f32" else "prefill_7b_bf16"
    w = I.workload(name, d_qk=dk, d_v=dv)
    d = I.gen_prefill(w, pairs=_pairs(rng, w, P), T=T)
    if state:
        d["C0"], d["n0"], d["m0"] = _random_state(rng, P, dk, dv)
    else:
        d["C0"] = d["n0"] = d["m0"] = None
    dh = I.to_io_dtype(rng.normal(0.0, 1.0, (P, T, dv)), io)
    gpu, ref = bwd_gpu(d, dh, state), list(bwd_oracle(d, dh))
    if not state:
        # From the zero state the first token's read-out is sigma(o~) (q.k) v /
        # max(|q.k|, e^{-m}): where the floor is inactive it does not change
        # when q is scaled, so dq of that token is exactly zero (the oracle
        # gives ~1e-16) and a per-row ratio would divide float32 rounding by
        # it.  That row is held to the gradient's global scale instead.
        scale = float(np.abs(ref[0]).max())
        first = float(np.abs(gpu[0][:, :1] - ref[0][:, :1]).max())
        assert first <= PT.TOL[io] * scale, (f"bwd sweep {i}", "dq token 0", first, scale)
        gpu = [gpu[0][:, 1:]] + list(gpu[1:])
        ref = [ref[0][:, 1:]] + ref[1:]
    bwd_compare(gpu, ref, io, f"bwd sweep {i}", state_grad=state)


@pytest.mark.parametrize("i", range(N_LAYER))
def test_layer_sweep(i):
    rng = _draw(7700 + i)
    io = ("f32", "bf16")[int(rng.integers(2))]
    H = int(rng.integers(1, 5))
    dk = 16 * int(rng.integers(1, 17))
    dv = 16 * int(rng.integers(1, 33))
    d_model = 8 * int(rng.integers(4, 65))
    B = int(rng.integers(1, 4))
    T = int(rng.integers(1, 301))
    chunk = int(rng.choice([16, 32, 64, 128]))
    state = bool(rng.integers(2))
    print(f"[case] layer sweep {i}: io={io} B={B} T={T} d_model={d_model} H={H} dk={dk} dv={dv} "
          f"chunk={chunk} state={state}", flush=True)
    init = I.layer_workload("layer_small").init_state if state else None
    w = I.layer_workload("layer_small", io=io, B=B, T=T, d_model=d_model, H=H, d_qk=dk, d_v=dv, chunk=chunk,
                         init_state=init)
    d = I.gen_layer(w)
    layer_compare(layer_gpu(d, chunk), layer_oracle(d, io), io, f"layer sweep {i}")


@pytest.mark.parametrize("i", range(N_SLSTM))
def test_slstm_sweep(i):
    rng = _draw(7900 + i)
    io = ("f32", "bf16")[int(rng.integers(2))]
    d = 16 * int(rng.integers(1, 9))
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 5))
    T = int(rng.integers(1, 301))
    state = bool(rng.integers(2))
    print(f"[case] slstm sweep {i}: io={io} B={B} H={H} T={T} d={d} state={state}", flush=True)
    w = I.slstm_workload("slstm_small", io=io, B=B, H=H, T=T, d=d, state=state)
    g = I.gen_slstm(w)
    slstm_compare(slstm_gpu(g), slstm_oracle(g), io, f"slstm sweep {i}")
