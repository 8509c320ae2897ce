"""GPU parity of the backward (mlstm_bwd_chunkwise) against the float64
oracle's backward, on seeded workloads and their edge cases.

The error metric is the forward's (tests/parity.py): per row, max |x - r| /
max |r|, maximised over rows.  A row is one token's d_qk or d_v vector for
dq, dk, dv and do, one sequence's vector over T for di and df, one pair's
dC0 or dn0, and the pairs' dm0 together."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity as PT
from xlstm_mlstm_matrix_amd import binding, inputs as I

pytestmark = pytest.mark.gpu


def case(name, pairs=None, T=None, **override):
    w = I.workload(name, **override)
    d = I.gen_prefill(w, pairs=pairs, T=T)
    P, T_, _ = d["q"].shape
    rng = np.random.default_rng(4242 + T_)
    dh = I.to_io_dtype(rng.normal(0.0, 1.0, (P, T_, w.d_v)), w.io)
    return w, d, dh


def run_gpu(d, dh, state_grad):
    g = PT.cuda(d)
    add = lambda t: None if t is None else t.unsqueeze(0)
    out = binding.bwd_chunkwise(add(g["q"]), add(g["k"]), add(g["v"]), add(g["i_pre"]), add(g["f_pre"]),
                                add(g["o_pre"]), add(dh.cuda()), add(g["C0"]), add(g["n0"]), add(g["m0"]),
                                state_grad=state_grad)
    torch.cuda.synchronize()
    return [PT.to_np(x[0]) for x in out]


def run_oracle(d, dh):
    st = (d["C0"], d["n0"], d["m0"]) if d["C0"] is not None else (None, None, None)
    return oracle.backward(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"], dh, *st)


NAMES = ["dq", "dk", "dv", "di", "df", "do", "dC0", "dn0", "dm0"]


def compare(gpu, ref, io, what, state_grad=True, global_norm=()):
    """global_norm: gradients compared by the global infinity-norm ratio
    max |x - r| / max |r| over the whole tensor instead of per row."""
    tol = PT.TOL[io]
    errs = {}
    for j, name in enumerate(NAMES[:len(gpu)]):
        x, r = gpu[j], ref[j]
        assert np.all(np.isfinite(x)), (what, name, "non-finite")
        if name in ("dC0",):
            x, r = x.reshape(x.shape[0], -1), r.reshape(r.shape[0], -1)
        if name == "dm0" or name in global_norm:
            x, r = x.reshape(1, -1), r.reshape(1, -1)
        errs[name] = PT.row_relerr(x, r)
    print(f"[parity] {what}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v <= tol, (what, k, v)


def test_tiny_f32():
    """B=1 H=1 T=64 d=16 float32 from the zero state (two 32-token chunks)."""
    w, d, dh = case("tiny_f32")
    compare(run_gpu(d, dh, True), run_oracle(d, dh), "f32", "tiny")


@pytest.mark.parametrize("T", [1, 31, 32, 33, 100])
def test_small_f32_ragged(T):
    """d_qk = d_v = 64, float32, a random initial state, lengths that end
    inside or at the border of a chunk; the initial state's gradients too."""
    w, d, dh = case("small_f32", pairs=[(0, 1), (3, 2)], T=T)
    compare(run_gpu(d, dh, True), run_oracle(d, dh), "f32", f"small T={T}")


def test_small_f32_full_length():
    """The small workload's full T = 1024 on a subset of its pairs."""
    w, d, dh = case("small_f32", pairs=[(1, 1), (2, 3)])
    compare(run_gpu(d, dh, True), run_oracle(d, dh), "f32", "small T=1024")


@pytest.mark.parametrize("dk,dv", [(16, 64), (64, 16), (32, 48), (48, 32)])
def test_head_dims(dk, dv):
    w, d, dh = case("small_f32", pairs=[(0, 0)], T=90, d_qk=dk, d_v=dv)
    compare(run_gpu(d, dh, True), run_oracle(d, dh), "f32", f"dk={dk} dv={dv}")


def test_bf16_io():
    """bfloat16 inputs and dh (the 7B-layer distributions at d = 64); the
    gradients are float32 and compared with the oracle run on the same
    rounded inputs."""
    w, d, dh = case("prefill_7b_bf16", pairs=[(0, 0), (5, 3)], T=200, d_qk=64, d_v=64)
    compare(run_gpu(d, dh, False), run_oracle(d, dh)[:6], "bf16", "bf16 io", state_grad=False)


def test_gate_spikes():
    """Input gates of +-30 and a forget gate near one: the stabilizer moves
    by tens within a chunk.  dq is compared by the global norm: where the
    normalizer's floor is inactive h does not change when q is scaled, so dq
    = C a + n beta is orthogonal to q, and after a dominant input gate the
    memory is nearly rank one (C ~ k v^T, n ~ k) and the two terms cancel to
    a tiny remainder -- its per-row ratio would measure float32 cancellation,
    not the kernel.  Every other gradient keeps the per-row metric."""
    w, d, dh = case("small_f32", pairs=[(2, 2)], T=150)
    i = d["i_pre"].clone()
    i[:, 10] = 30.0
    i[:, 70] = 25.0
    i[:, 100:110] = -30.0
    d["i_pre"] = i
    d["f_pre"][:, 120:] = -1e-4
    compare(run_gpu(d, dh, True), run_oracle(d, dh), "f32", "spikes", global_norm=("dq",))


def test_matches_autograd_free_identities():
    """Independent of the oracle: di = k . dk and df is the reverse
    cumulative sum of q . dq - k . dk, on the GPU's own outputs."""
    w, d, dh = case("small_f32", pairs=[(1, 2)], T=130)
    dq, dk, dv, di, df, do = (x[0] for x in run_gpu(d, dh, False))  # the one pair
    q, k = (d[x][0].double().numpy() for x in ("q", "k"))
    np.testing.assert_allclose(di, (k * dk).sum(-1), rtol=1e-4, atol=1e-4 * np.abs(di).max())
    x = (q * dq).sum(-1) - (k * dk).sum(-1)
    rev = np.cumsum(x[::-1])[::-1]
    np.testing.assert_allclose(df, rev, rtol=1e-3, atol=1e-3 * np.abs(df).max())


@pytest.mark.parametrize("dk,dv,io", [(128, 64, "f32"), (64, 128, "f32"), (80, 96, "f32"),
                                      (256, 512, "f32"), (256, 512, "bf16"),
                                      # odd counts of 16-row tiles above 128 (the second row
                                      # tile of a wavefront valid on some only) and a last
                                      # value-column block of 16 of 128 columns
                                      (240, 400, "f32"), (176, 144, "bf16")])
def test_large_heads(dk, dv, io):
    """Heads above 64 (state and tiles in the workspace), with a random initial
    state and a ragged last chunk."""
    w, d, dh = case("small_f32", pairs=[(0, 1), (2, 3)], T=70, d_qk=dk, d_v=dv, io=io)
    out = run_gpu(d, dh, io == "f32")
    ref = run_oracle(d, dh)
    compare(out, ref[:len(out)], io, f"large heads {dk}x{dv} {io}", state_grad=io == "f32")


@pytest.mark.parametrize("T", [1, 32, 33])
def test_large_heads_chunk_edges(T):
    """Heads above 64 at one token, exactly one chunk and one token past it
    (the scans' single-chunk and one-token-chunk cases)."""
    w, d, dh = case("small_f32", pairs=[(0, 1), (1, 0)], T=T, d_qk=128, d_v=192, io="f32")
    out = run_gpu(d, dh, True)
    ref = run_oracle(d, dh)
    compare(out, ref[:len(out)], "f32", f"large heads T={T}", state_grad=True)


def test_7b_heads_bf16():
    """The 7B layer's heads and distributions (bf16, d_qk 256, d_v 512) over
    200 tokens of two pairs, from the zero state."""
    w, d, dh = case("prefill_7b_bf16", pairs=[(0, 0), (7, 5)], T=200)
    compare(run_gpu(d, dh, False), run_oracle(d, dh)[:6], "bf16", "7b heads", state_grad=False)


@pytest.mark.parametrize("T,pairs", [(1024, [(0, 0), (7, 5)]), (2100, [(3, 6)])])
def test_7b_heads_bf16_long(T, pairs):
    """The 7B layer's heads (bf16, d_qk 256, d_v 512) over long sequences:
    1024 tokens (32 chunks) of two pairs, and 2100 tokens of one pair, which
    crosses the 64-chunk groups of the carried-gradient scan (the benchmark
    runs 4096 tokens, 128 chunks)."""
    w, d, dh = case("prefill_7b_bf16", pairs=pairs, T=T)
    print(f"[case] backward 7b heads T={T} pairs={pairs}", flush=True)
    out = run_gpu(d, dh, False)
    compare(out, run_oracle(d, dh)[:6], "bf16", f"7b heads T={T}", state_grad=False)


def test_long_sequence_f32_chunk_groups():
    """Float32, d=64, 2200 tokens (69 chunks of 32) with an initial state:
    the carried-gradient scan runs past its first 64-chunk group, with the
    state gradients."""
    w = I.workload("small_f32", T=2200)   # the workload's own T is 1024
    d = I.gen_prefill(w, pairs=[(2, 1)])
    dh = I.to_io_dtype(np.random.default_rng(4242 + 2200).normal(0.0, 1.0, (1, 2200, w.d_v)), w.io)
    assert d["q"].shape[1] == 2200
    compare(run_gpu(d, dh, True), run_oracle(d, dh), "f32", "f32 T=2200")


def test_unsupported_head_dim_raises():
    w, d, dh = case("small_f32", pairs=[(0, 0)], T=40, d_qk=272, d_v=64)
    with pytest.raises(binding.MlstmError):
        run_gpu(d, dh, False)
