"""GPU parity of the recurrent step (mlstm_step) against the float64 oracle,
and of a run of steps against the chunkwise forward over the same tokens."""
import numpy as np
import pytest
import torch

import oracle
from tests import parity as PT
from xlstm_mlstm_matrix_amd import binding, inputs as I

pytestmark = pytest.mark.gpu


def run_steps(steps, state, inplace=True, split=True):
    """steps: dict of [S, B, H, ...] device tensors; state: (C, n, m) or None.
    With ``split`` every step uses the row-split kernel where the shape has
    one, all through one workspace."""
    S, B, H = steps["q"].shape[:3]
    dk, dv = steps["q"].shape[-1], steps["v"].shape[-1]
    ws = binding.step_workspace(B, H, dk, dv, steps["q"].dtype, steps["q"].device) if split else None
    C = n = m = None
    if state is not None:
        C, n, m = (x.clone() for x in state)
    hs = []
    for t in range(S):
        h, C, n, m = binding.step(*(steps[k][t] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")),
                                  C, n, m, inplace=inplace, split=split, workspace=ws)
        hs.append(h)
    torch.cuda.synchronize()
    return torch.stack(hs, dim=2), C, n, m  # h: [B, H, S, d_v]


def oracle_steps(steps, state):
    """The oracle over the same S tokens, per pair: inputs rearranged to [P, S, ...]."""
    S, B, H = steps["q"].shape[:3]
    P = B * H
    tr = lambda t: t.reshape(S, P, *t.shape[3:]).transpose(0, 1).contiguous()
    st = (None, None, None)
    if state is not None:
        st = tuple(x.reshape(P, *x.shape[2:]) for x in state)
    return oracle.forward(*(tr(steps[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")), *st)


def compare_steps(gpu, ref, io, what):
    h, C, n, m = gpu
    B, H = h.shape[:2]
    P = B * H
    flat = lambda t: t.reshape(P, *t.shape[2:])
    PT.compare_fwd((flat(h), flat(C), flat(n), flat(m)), ref, io, what)


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 64), (64, 128), (256, 512), (48, 80),
                                   (80, 512), (208, 512), (256, 256), (144, 272)])
def test_steps_vs_oracle(io, dk, dv, split):
    """Head shapes with one row block (no split), with several (256 x 512: 4
    blocks of 64 rows; 256 x 256: 2 of 128) and with a ragged last block (80
    and 208 rows in blocks of 64; 144 rows in blocks of 112 at d_v = 272)."""
    w = I.workload("decode_bf16", io=io, d_qk=dk, d_v=dv)
    steps = PT.cuda(I.gen_decode_steps(w, range(24), B=3))
    state = tuple(x.cuda() for x in I.gen_decode_state(w, B=3))
    compare_steps(run_steps(steps, state, split=split), oracle_steps(steps, state), io,
                  f"step {io} {dk}x{dv} split={split}")


def test_split_matches_one_workgroup():
    """The row split sums the same products in another order: it agrees with
    the one-workgroup kernel to rounding, over a run of in-place steps."""
    w = I.workload("decode_bf16", io="f32")
    steps = PT.cuda(I.gen_decode_steps(w, range(12), B=2))
    state = tuple(x.cuda() for x in I.gen_decode_state(w, B=2))
    a = run_steps(steps, state, split=True)
    b = run_steps(steps, state, split=False)
    for x, y in zip(a, b):
        scale = y.abs().max().item()
        assert (x - y).abs().max().item() <= 1e-5 * scale, (x - y).abs().max().item()


def test_workspace_is_scratch():
    """The workspace needs no initial contents (filled with NaN here) and one
    buffer serves calls of different shapes in stream order."""
    ws = binding.step_workspace(3, 8, 256, 512, torch.bfloat16, "cuda")
    ws.view(torch.float32).fill_(float("nan"))
    for dk, dv, B in ((256, 512, 3), (80, 512, 2), (256, 256, 3), (208, 512, 1), (256, 512, 2)):
        w = I.workload("decode_bf16", d_qk=dk, d_v=dv)
        steps = PT.cuda(I.gen_decode_steps(w, range(3), B=B))
        state = tuple(x.cuda() for x in I.gen_decode_state(w, B=B))
        C, n, m = (x.clone() for x in state)
        hs = []
        for t in range(3):
            h, C, n, m = binding.step(*(steps[k][t] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")),
                                      C, n, m, workspace=ws)
            hs.append(h)
        torch.cuda.synchronize()
        compare_steps((torch.stack(hs, dim=2), C, n, m), oracle_steps(steps, state), "bf16",
                      f"shared workspace {dk}x{dv} B={B}")


def test_inplace_equals_out_of_place_bitwise():
    w = I.workload("decode_bf16", d_qk=256, d_v=512)
    steps = PT.cuda(I.gen_decode_steps(w, range(6), B=4))
    state = tuple(x.cuda() for x in I.gen_decode_state(w, B=4))
    a = run_steps(steps, state, inplace=True)
    b = run_steps(steps, state, inplace=False)
    c = run_steps(steps, state, inplace=True)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(x, z)


def test_steps_equal_chunkwise():
    """1 token at a time through mlstm_step == the chunkwise forward over the
    same tokens from the same state (both also against the oracle)."""
    w = I.workload("decode_bf16")
    S, Bq = 160, 2
    steps = PT.cuda(I.gen_decode_steps(w, range(S), B=Bq))
    state = tuple(x.cuda() for x in I.gen_decode_state(w, B=Bq))
    gs = run_steps(steps, state)
    seq = {k: v.permute(1, 2, 0, *range(3, v.dim())).contiguous() for k, v in steps.items()}  # [B,H,S,...]
    h, (C, n, m) = binding.fwd_chunkwise(*(seq[k] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")),
                                         *state, chunk=64, variant="fused")
    torch.cuda.synchronize()
    ref = oracle_steps(steps, state)
    compare_steps(gs, ref, "bf16", "steps")
    compare_steps((h, C, n, m), ref, "bf16", "chunkwise over the same tokens")


def test_decode_full_size():
    """The decode workload at full size (B=256 H=8 d_qk=256 d_v=512, 1024
    consecutive in-place steps, the launch configuration the benchmark times).
    The oracle runs every pair over all steps (in batches of 128 pairs): the
    final (C, n, m) of all 2048 pairs is compared, h of every step on 64
    sampled pairs (every 32nd), and every pair's final stabilizer against its
    closed form."""
    w = I.workload("decode_bf16")
    S = w.T
    P = w.B * w.H
    print("[case] decode full size: generating inputs", flush=True)
    C, n, m = (x.cuda() for x in I.gen_decode_state(w))
    C0s, n0s, m0s = (x.reshape(P, *x.shape[2:]) for x in I.gen_decode_state(w))  # CPU copies
    hs_sample = []
    pairs = np.arange(0, P, 32)
    steps_cpu = []
    chunk = 64
    ws = binding.step_workspace(w.B, w.H, w.d_qk, w.d_v, torch.bfloat16, C.device)
    keys = ("q", "k", "v", "i_pre", "f_pre", "o_pre")
    for t0 in range(0, S, chunk):
        st_cpu = I.gen_decode_steps(w, range(t0, min(S, t0 + chunk)), threads=16)
        st = PT.cuda(st_cpu)
        for t in range(st["q"].shape[0]):
            h, C, n, m = binding.step(*(st[k][t] for k in keys), C, n, m, workspace=ws)
            hs_sample.append(h.reshape(P, -1)[pairs].cpu())
        steps_cpu.append({k: v.reshape(v.shape[0], P, *v.shape[3:]) for k, v in st_cpu.items()})
        print(f"[case] decode steps done: {min(S, t0 + chunk)}", flush=True)
    torch.cuda.synchronize()
    assert torch.isfinite(C).all() and torch.isfinite(n).all()
    Cg, ng, mg = C.reshape(P, 256, 512).cpu(), n.reshape(P, 256).cpu(), m.reshape(P).cpu()
    del C, n, m
    torch.cuda.empty_cache()
    gi = torch.cat([c["i_pre"] for c in steps_cpu]).T.double().numpy()   # [P, S]
    gf = torch.cat([c["f_pre"] for c in steps_cpu]).T.double().numpy()
    m_ref_all = PT.m_closed_form(gi, gf, m0s.double().numpy())
    assert np.max(np.abs(PT.to_np(mg) - m_ref_all)) <= PT.TOL_M["bf16"]
    hg = torch.stack(hs_sample, dim=1)   # [64, S, d_v]
    worst = [0.0, 0.0, 0.0, 0.0]
    nb = 128
    for p0 in range(0, P, nb):
        sel = slice(p0, p0 + nb)
        seq = {k: torch.cat([c[k][:, sel] for c in steps_cpu]).transpose(0, 1).contiguous() for k in keys}
        ref = oracle.forward(*(seq[k] for k in keys), C0s[sel], n0s[sel], m0s[sel], threads=16)
        del seq
        # h of the sampled pairs in this batch; state of every pair in it
        mine = [j for j, p in enumerate(pairs) if p0 <= p < p0 + nb]
        rows = [int(pairs[j]) - p0 for j in mine]
        # only the sampled pairs' h was kept from the GPU: the other rows of
        # this batch take the oracle's own h, so the h check covers exactly
        # the sampled pairs
        h_b = torch.from_numpy(ref[0].copy())
        h_b[rows] = hg[mine].double()
        errs = PT.compare_fwd((h_b, Cg[sel], ng[sel], mg[sel]), ref, "bf16",
                              f"decode full size, pairs {p0}..{p0 + nb - 1}")
        worst = [max(a, b) for a, b in zip(worst, errs)]
        print(f"[case] decode oracle batch {p0 // nb + 1}/{P // nb} done", flush=True)
    print(f"[parity] decode full size, all {P} pairs: h (64 sampled) {worst[0]:.2e}  C {worst[1]:.2e}  "
          f"n {worst[2]:.2e}  m {worst[3]:.2e}", flush=True)
