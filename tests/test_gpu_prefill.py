"""GPU parity of the chunkwise forward (mlstm_fwd_chunkwise) against the
float64 oracle, on the seeded workloads and their edge cases."""
import numpy as np
import pytest
import torch

from tests import parity as PT
from xlstm_mlstm_matrix_amd import binding, inputs as I

pytestmark = pytest.mark.gpu


def case(name, pairs=None, T=None, **override):
    w = I.workload(name, **override)
    return w, I.gen_prefill(w, pairs=pairs, T=T)


def test_tiny_f32():
    """B=1 H=1 T=64 d_qk=d_v=16 chunk=16 float32, zero initial state."""
    w, d = case("tiny_f32")
    PT.compare_fwd(PT.run_gpu_fwd(d, w.chunk), PT.run_oracle(d), "f32", "tiny_f32")


def test_small_f32():
    """B=4 H=4 T=1024 d=64 chunk=64 float32 with a random initial state (every pair)."""
    w, d = case("small_f32")
    PT.compare_fwd(PT.run_gpu_fwd(d, w.chunk), PT.run_oracle(d), "f32", "small_f32")


@pytest.mark.parametrize("T", [1, 15, 31, 32, 33, 61, 64, 65, 127, 128, 129, 200, 512])
def test_7b_shapes_ragged(T):
    """d_qk=256, d_v=512 bf16 at lengths that end mid-chunk or inside one chunk."""
    w, d = case("prefill_7b_bf16", pairs=[(0, 0), (5, 3)], T=T)
    PT.compare_fwd(PT.run_gpu_fwd(d, 64, variant="fused"), PT.run_oracle(d), "bf16", f"7b T={T}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_invariance_bf16(chunk):
    """The chunk length is a schedule choice only: every chunk matches the oracle."""
    w, d = case("prefill_7b_bf16", pairs=[(1, 2)], T=300)
    PT.compare_fwd(PT.run_gpu_fwd(d, chunk, variant="fused"), PT.run_oracle(d), "bf16", f"chunk {chunk}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunk_invariance_f32(chunk):
    w, d = case("small_f32", pairs=[(0, 1), (3, 3)], T=333)
    PT.compare_fwd(PT.run_gpu_fwd(d, chunk, variant="fused"), PT.run_oracle(d), "f32", f"f32 chunk {chunk}")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 48), (64, 64), (96, 160), (128, 128), (256, 512)])
def test_head_dims(dk, dv):
    """Supported head dimensions (multiples of 16), both I/O dtypes."""
    for io in ("f32", "bf16"):
        w, d = case("prefill_7b_bf16", pairs=[(2, 2)], T=130, d_qk=dk, d_v=dv, io=io)
        PT.compare_fwd(PT.run_gpu_fwd(d, 32, variant="fused"), PT.run_oracle(d), io, f"{io} dk={dk} dv={dv}")


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 256), (256, 128), (256, 384)])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("variant", ["fused", "segscan"])
def test_chunk64_value_blocks(dk, dv, with_state, variant):
    """Chunk 64 with d_v a multiple of 128 (128-column value blocks), each d_qk
    in {64, 128, 256}, ragged T, from the zero state and from a random one; one
    pass, and the segmented schedule (2 segments at T=200: the state-only pass,
    the combine with the initial state, the seeded output pass)."""
    w, d = case("prefill_7b_bf16", pairs=[(1, 1), (6, 3)], T=200, d_qk=dk, d_v=dv)
    if with_state:
        rng = np.random.default_rng(1000 + dk + dv)
        P = d["q"].shape[0]
        d["C0"] = torch.from_numpy(rng.normal(0.0, 0.05, (P, dk, dv))).float()
        d["n0"] = torch.from_numpy(rng.normal(0.0, 0.05, (P, dk))).float()
        d["m0"] = torch.from_numpy(rng.uniform(-1.0, 1.0, P)).float()
    PT.compare_fwd(PT.run_gpu_fwd(d, 64, variant=variant), PT.run_oracle(d), "bf16",
                   f"chunk 64 dk={dk} dv={dv} state={with_state} {variant}")


@pytest.mark.parametrize("variant", ["fused", "segscan"])
@pytest.mark.parametrize("dk,dv,io", [(16, 432, "bf16"), (32, 176, "f32"), (64, 320, "bf16"),
                                      (16, 64, "f32"), (48, 96, "bf16"), (64, 512, "bf16")])
def test_chunk128_small_heads(dk, dv, io, variant):
    """Chunk 128 runs as such only where its tiles fit in LDS, at d_qk up to
    64: a chunk then spans two 64-token parts of the gate scan, whose running
    sum of f~ and prefix maximum of u carry from the first part into the
    second.  Five whole chunks and a ragged last one, from a random state;
    the segmented schedule cuts them into 3 segments."""
    name = "small_f32" if io == "f32" else "prefill_7b_bf16"
    T = 700
    w, d = case(name, pairs=[(0, 1), (1, 0), (2, 3)], T=T, d_qk=dk, d_v=dv)
    rng = np.random.default_rng(128 + dk + dv)
    d["C0"] = torch.from_numpy(rng.normal(0.0, 0.05, (3, dk, dv))).float()
    d["n0"] = torch.from_numpy(rng.normal(0.0, 0.05, (3, dk))).float()
    d["m0"] = torch.from_numpy(rng.uniform(-1.0, 1.0, 3)).float()
    kc, nseg = binding.schedule(1, 3, T, dk, dv, 128, binding.BF16 if io == "bf16" else binding.F32, variant)
    assert kc == 128 and nseg == (3 if variant == "segscan" else 1)
    PT.compare_fwd(PT.run_gpu_fwd(d, 128, variant=variant), PT.run_oracle(d), io,
                   f"chunk 128 dk={dk} dv={dv} {io} {variant}")


@pytest.mark.parametrize("dk", [64, 128, 256])
@pytest.mark.parametrize("chunk", [32, 64])
def test_readout_keeps_state_precision(dk, chunk):
    """The inter-chunk read-out C'^T q must keep the float32 state's precision
    beyond bf16.  Every row of C0 is a common vector plus a per-row offset
    2^-9 times smaller, and q_t = e_a - e_b picks the difference of two rows,
    so h is the difference of the two offsets: a read-out that rounds C' to
    bf16 alone (8 significant bits) loses it whole, the high part plus the
    rounded remainder keeps it to well inside the tolerance.  k = 0 keeps the
    intra-chunk part and the update at zero; i~ = -30 keeps the stabilizer at
    m, so the read-out is all that h holds."""
    P, T, dv = 2, 150, 128
    rng = np.random.default_rng(77 + dk + chunk)
    q = np.zeros((P, T, dk))
    for p in range(P):
        for t in range(T):
            a, b = rng.choice(dk, size=2, replace=False)
            q[p, t, a], q[p, t, b] = 1.0, -1.0
    common = rng.normal(0.0, 1.0, (P, 1, dv))
    C0 = common + rng.normal(0.0, 2.0 ** -9, (P, dk, dv))
    d = {
        "q": torch.from_numpy(q).to(torch.bfloat16),
        "k": torch.zeros((P, T, dk), dtype=torch.bfloat16),
        "v": torch.from_numpy(rng.normal(0.0, 1.0, (P, T, dv))).to(torch.bfloat16),
        "i_pre": torch.full((P, T), -30.0, dtype=torch.float32),
        "f_pre": torch.from_numpy(-np.log1p(np.exp(-rng.normal(5.0, 1.0, (P, T))))).float(),
        "o_pre": torch.from_numpy(rng.normal(0.0, 1.0, (P, T, dv))).to(torch.bfloat16),
        "C0": torch.from_numpy(C0).float(),
        "n0": torch.from_numpy(rng.normal(0.0, 1.0, (P, dk))).float(),
        "m0": torch.zeros((P,), dtype=torch.float32),
    }
    gpu = PT.run_gpu_fwd(d, chunk, variant="fused")
    ref = PT.run_oracle(d)
    eh = PT.compare_fwd(gpu, ref, "bf16", f"read-out precision dk={dk} chunk={chunk}")[0]
    # bf16 alone would be off by more than 50% on every token (emulated on
    # the CPU); the high part plus the remainder stays under 0.6%
    assert eh <= 2e-2


def test_segscan_equals_oracle():
    """The segmented schedule (local states, scan, seeded pass) on bf16."""
    w, d = case("prefill_7b_bf16", pairs=[(0, 1), (4, 4)], T=1000)
    gpu = PT.run_gpu_fwd(d, 64, variant="segscan")
    ref = PT.run_oracle(d)
    PT.compare_fwd(gpu, ref, "bf16", "segscan")
    fused = PT.run_gpu_fwd(d, 64, variant="fused")
    PT.compare_fwd(fused, ref, "bf16", "fused (same inputs)")


def test_segscan_with_initial_state_f32():
    w, d = case("small_f32", pairs=[(1, 1), (2, 0)], T=900)
    PT.compare_fwd(PT.run_gpu_fwd(d, 32, variant="segscan"), PT.run_oracle(d), "f32", "segscan f32 + state")


@pytest.mark.parametrize("dk,dv,T,with_state", [(256, 512, 748, False), (256, 512, 837, True),
                                                (128, 256, 1100, False), (64, 128, 900, True)])
def test_segscan_multi_chunk_segments(dk, dv, T, with_state):
    """The segmented schedule with several chunks per segment and a ragged last
    one.  Sixteen pairs give the planner enough column-block workgroups that it
    cuts 4 to 6 segments of 3 or 4 chunks each.  The state-only pass then walks
    several chunks per segment (the other segmented cases have 2, or 128 at the
    long-context size), and the combine chains 3 to 5 local states.  Checked from
    the zero state and from a random one."""
    pairs = [(b, h) for b in range(2) for h in range(8)]
    w, d = case("prefill_7b_bf16", pairs=pairs, T=T, d_qk=dk, d_v=dv)
    if with_state:
        rng = np.random.default_rng(2000 + T)
        P = len(pairs)
        d["C0"] = torch.from_numpy(rng.normal(0.0, 0.05, (P, dk, dv))).float()
        d["n0"] = torch.from_numpy(rng.normal(0.0, 0.05, (P, dk))).float()
        d["m0"] = torch.from_numpy(rng.uniform(-1.0, 1.0, P)).float()
    kc, nseg = binding.schedule(1, len(pairs), T, dk, dv, 64, binding.BF16, "segscan")
    cps = -(-T // (64 * nseg))  # chunks per segment: segments are whole chunks, nseg of them cover T
    print(f"[case] segscan dk={dk} dv={dv} T={T} segments={nseg} chunks/segment={cps}", flush=True)
    assert kc == 64 and nseg >= 4 and cps >= 3
    PT.compare_fwd(PT.run_gpu_fwd(d, 64, variant="segscan"), PT.run_oracle(d), "bf16",
                   f"segscan dk={dk} dv={dv} T={T} state={with_state}")


def test_state_carry():
    """fwd(x[:t0]) then fwd(x[t0:], state) equals fwd(x) and the oracle."""
    w, d = case("small_f32", pairs=[(0, 0), (1, 3)], T=700)
    ref = PT.run_oracle(d)
    t0 = 257
    first = {k: (v[:, :t0].contiguous() if v is not None and v.dim() >= 2 and k not in ("C0", "n0") else v)
             for k, v in d.items()}
    first["m0"] = d["m0"]
    h1, C1, n1, m1 = PT.run_gpu_fwd(first, 64)
    second = {k: (v[:, t0:].contiguous() if v is not None and v.dim() >= 2 and k not in ("C0", "n0") else v)
              for k, v in d.items()}
    second["C0"], second["n0"], second["m0"] = C1.cpu(), n1.cpu(), m1.cpu()
    h2, C2, n2, m2 = PT.run_gpu_fwd(second, 64)
    PT.compare_fwd((torch.cat([h1, h2], dim=1), C2, n2, m2), ref, "f32", "split at 257")


def test_inplace_state_bitwise_and_deterministic():
    """C_T == C0 (in place) gives bitwise the same result as separate buffers,
    and repeated runs are bitwise identical."""
    w = I.workload("small_f32")
    d = PT.cuda(I.gen_prefill(w, pairs=[(0, 0), (1, 1), (2, 2)], T=300))
    add = lambda t: t.unsqueeze(0)
    args = [add(d[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    C0, n0, m0 = add(d["C0"]), add(d["n0"]), add(d["m0"])
    for variant in ("fused", "segscan"):
        h1, (C1, n1, m1) = binding.fwd_chunkwise(*args, C0, n0, m0, chunk=64, variant=variant)
        h2, (C2, n2, m2) = binding.fwd_chunkwise(*args, C0, n0, m0, chunk=64, variant=variant)
        Ci, ni, mi = C0.clone(), n0.clone(), m0.clone()
        h3, _ = binding.fwd_chunkwise(*args, Ci, ni, mi, chunk=64, variant=variant,
                                      C_T=Ci, n_T=ni, m_T=mi)
        torch.cuda.synchronize()
        for a, b in ((h1, h2), (C1, C2), (n1, n2), (m1, m2), (h1, h3), (C1, Ci), (n1, ni), (m1, mi)):
            assert torch.equal(a, b), variant


def test_outputs_fully_written():
    """Outputs pre-filled with NaN come back finite (no element left unwritten)."""
    w, d = case("prefill_7b_bf16", pairs=[(3, 3)], T=77)
    g = PT.cuda(d)
    add = lambda t: t.unsqueeze(0)
    h = torch.full((1, 1, 77, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    C = torch.full((1, 1, 256, 512), float("nan"), device="cuda")
    n = torch.full((1, 1, 256), float("nan"), device="cuda")
    m = torch.full((1, 1), float("nan"), device="cuda")
    binding.fwd_chunkwise(*[add(g[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")],
                          chunk=64, h=h, C_T=C, n_T=n, m_T=m)
    torch.cuda.synchronize()
    for t in (h, C, n, m):
        assert torch.isfinite(t).all()


def test_input_gate_spikes():
    """Input-gate pre-activations of +-50 (e^50 overflows nothing in the
    stabilized form) and a forget gate near 1."""
    w, d = case("prefill_7b_bf16", pairs=[(0, 0), (1, 1)], T=150)
    i = d["i_pre"].clone()
    i[:, 10] = 50.0
    i[:, 90] = 45.0
    i[:, 100:110] = -50.0
    d["i_pre"] = i
    d["f_pre"][:, 120:] = -1e-4
    PT.compare_fwd(PT.run_gpu_fwd(d, 64, variant="fused"), PT.run_oracle(d), "bf16", "spikes")


def test_linear_attention_special_case():
    """i~ = f~ = 0 from the zero state: num = tril(Q K^T) V (unnormalized causal
    linear attention), checked on the GPU against that closed form directly."""
    w, d = case("small_f32", pairs=[(0, 0)], T=96)
    d["i_pre"].zero_()
    d["f_pre"].zero_()
    d["C0"] = d["n0"] = d["m0"] = None
    h, C, n, m = PT.run_gpu_fwd(d, 32, variant="fused")
    q, k, v, o = (d[x][0].double().numpy() for x in ("q", "k", "v", "o_pre"))
    A = np.tril(q @ k.T)
    den = np.maximum(np.abs(A.sum(axis=1)), 1.0)
    num = PT.to_np(h) / (1.0 / (1.0 + np.exp(-o))) * den[:, None]
    assert PT.row_relerr(num, A @ v) <= PT.TOL["f32"]
    assert float(m.abs().max()) == 0.0


@pytest.fixture(scope="module")
def prefill_7b():
    """The 7B-layer-shaped workload (B=8 H=8 T=4096 d_qk=256 d_v=512, bf16)
    and its oracle result over every pair."""
    w = I.workload("prefill_7b_bf16")
    print("[case] 7b full size: inputs + oracle (64 pairs x 4096 tokens)", flush=True)
    d = I.gen_prefill(w, threads=16)
    ref = PT.run_oracle(d, threads=16)
    return w, d, ref


@pytest.mark.parametrize("variant", ["fused", "segscan"])
def test_7b_full_size(prefill_7b, variant):
    """The whole 7B-layer-shaped workload (chunk=64) in one call, in the
    launch configuration the benchmark times (fused) and as a segment scan:
    h of every token and the final (C, n, m) of every pair against the
    oracle; every pair's final stabilizer also against its closed form."""
    w, d, ref = prefill_7b
    print(f"[case] 7b full size, variant={variant}", flush=True)
    g = PT.cuda(d)
    shp = lambda t: t.reshape(w.B, w.H, *t.shape[1:])
    h, (C, n, m) = binding.fwd_chunkwise(*[shp(g[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")],
                                         chunk=w.chunk, variant=variant)
    torch.cuda.synchronize()
    del g
    m_ref = PT.m_closed_form(d["i_pre"].double().numpy(), d["f_pre"].double().numpy())
    assert np.max(np.abs(PT.to_np(m).reshape(-1) - m_ref)) <= PT.TOL_M["bf16"]
    flat = lambda t: t.reshape(w.B * w.H, *t.shape[2:])
    PT.compare_fwd((flat(h), flat(C), flat(n), flat(m)), ref, "bf16", f"7b full size {variant}, all 64 pairs")


@pytest.mark.parametrize("variant", ["fused", "segscan"])
def test_inplace_7b_heads_many_workgroups(variant):
    """In place (C_T == C0, n_T == n0, m_T == m0) at the 7B heads with 4
    value-column tiles per pair and 72 pairs (288 workgroups, more than the
    compute units): the tiles that read n0/m0 while another one writes n_T/m_T
    give bitwise the result of separate output buffers."""
    w = I.workload("prefill_7b_bf16", B=9)
    T = 200
    d = PT.cuda(I.gen_prefill(w, T=T, threads=16))
    wd = I.workload("decode_bf16")
    C0, n0, m0 = (x.cuda().reshape(-1, *x.shape[2:])[: w.B * w.H] for x in I.gen_decode_state(wd, B=w.B + 1))
    shp = lambda t: t.reshape(w.B, w.H, *t.shape[1:])
    args = [shp(d[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    st = [shp(C0), shp(n0), shp(m0)]
    h1, (C1, n1, m1) = binding.fwd_chunkwise(*args, *st, chunk=64, variant=variant)
    Ci, ni, mi = (x.clone() for x in st)
    h2, _ = binding.fwd_chunkwise(*args, Ci, ni, mi, chunk=64, variant=variant, C_T=Ci, n_T=ni, m_T=mi)
    torch.cuda.synchronize()
    for a, b, what in ((h1, h2, "h"), (C1, Ci, "C"), (n1, ni, "n"), (m1, mi, "m")):
        assert torch.equal(a, b), (variant, what)
    # and against the oracle on two pairs, one of them past the first 64
    idx = [5, 70]
    sub = {k: (v.reshape(w.B * w.H, *v.shape[2:])[idx].cpu() if v is not None else None)
           for k, v in zip(("q", "k", "v", "i_pre", "f_pre", "o_pre"), args)}
    sub.update(C0=C0[idx].cpu(), n0=n0[idx].cpu(), m0=m0[idx].cpu())
    flat = lambda t: t.reshape(w.B * w.H, *t.shape[2:])[idx]
    PT.compare_fwd((flat(h2), flat(Ci), flat(ni), flat(mi)), PT.run_oracle(sub), "bf16",
                   f"in place 7b heads {variant}")


@pytest.fixture(scope="module")
def long_context():
    """Long-context workload (B=1 H=8 T=65536 d_qk=256 d_v=512, bf16) and its
    oracle result over every pair."""
    w = I.workload("prefill_long_bf16")
    print("[case] long context: inputs + oracle (8 pairs x 65536 tokens)", flush=True)
    d = I.gen_prefill(w)
    ref = PT.run_oracle(d, threads=8)
    return w, d, ref


@pytest.mark.parametrize("variant", ["auto", "fused"])
def test_long_context_full_size(long_context, variant):
    """The long-context workload at full size, requested with chunk 128 (the
    kernels run 64-token chunks for d_qk 256), in the launch configuration
    the benchmark times (auto: segment scan) and as one fused pass: h of
    every token and the final (C, n, m) of every pair against the oracle."""
    w, d, ref = long_context
    kc, nseg = binding.schedule(w.B, w.H, w.T, w.d_qk, w.d_v, w.chunk, binding.BF16, variant)
    print(f"[case] long context variant={variant} kernel chunk={kc} segments={nseg}", flush=True)
    assert kc == 64 and (nseg > 1) == (variant == "auto")
    g = PT.cuda(d)
    shp = lambda t: t.reshape(w.B, w.H, *t.shape[1:])
    h, (C, n, m) = binding.fwd_chunkwise(*[shp(g[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")],
                                         chunk=w.chunk, variant=variant)
    torch.cuda.synchronize()
    flat = lambda t: t.reshape(w.B * w.H, *t.shape[2:])
    PT.compare_fwd((flat(h), flat(C), flat(n), flat(m)), ref, "bf16", f"long context {variant}")
    m_ref = PT.m_closed_form(d["i_pre"].double().numpy(), d["f_pre"].double().numpy())
    assert np.max(np.abs(PT.to_np(m).reshape(-1) - m_ref)) <= PT.TOL_M["bf16"]
