"""Out-of-bounds write checks on the GPU: every output and workspace of every
entry point is a view into a larger buffer whose guard regions (4 KiB before
and after) hold a sentinel bit pattern.  After the call the guards must be
bitwise unchanged, and the outputs (pre-filled with NaN) must be finite: no
kernel writes outside the extent the C ABI documents, and none leaves an
element unwritten."""
import math

import numpy as np
import pytest
import torch

from tests import parity as PT
from xlstm_mlstm_matrix_amd import binding, inputs as I

pytestmark = pytest.mark.gpu

GUARD_BYTES = 4096
PATTERN = {torch.bfloat16: (torch.int16, 0x7FA5), torch.float32: (torch.int32, 0x7FA5A5A5),
           torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """A tensor of ``shape`` at offset GUARD_BYTES inside a buffer whose other
    bytes (and, initially, the tensor itself) hold the sentinel pattern."""

    def __init__(self, shape, dtype):
        es = torch.tensor([], dtype=dtype).element_size()
        self.g = GUARD_BYTES // es
        n = math.prod(shape)
        self.buf = torch.empty(n + 2 * self.g, dtype=dtype, device="cuda")
        idt, pat = PATTERN[dtype]
        self.buf.view(idt).fill_(pat if idt != torch.int16 else np.int16(np.uint16(pat)).item())
        self.ref = self.buf[: self.g].clone()
        self.n = n
        self.t = self.buf[self.g: self.g + n].view(shape)

    def check(self, what, finite=True):
        torch.cuda.synchronize()
        head = self.buf[: self.g]
        tail = self.buf[self.g + self.n:]
        iv = PATTERN[self.buf.dtype][0]
        assert torch.equal(head.view(iv), self.ref.view(iv)), f"{what}: write before the buffer"
        assert torch.equal(tail.view(iv), self.ref.view(iv)), f"{what}: write past the buffer"
        if finite and self.buf.dtype != torch.uint8:
            assert torch.isfinite(self.t).all(), f"{what}: element left unwritten"


@pytest.mark.parametrize("variant", ["fused", "segscan"])
@pytest.mark.parametrize("T", [77, 130])
def test_prefill_guards(variant, T):
    w = I.workload("prefill_7b_bf16")
    d = PT.cuda(I.gen_prefill(w, pairs=[(0, 0), (2, 5), (6, 1)], T=T))
    P = 3
    add = lambda t: t.unsqueeze(0)
    h = Guarded((1, P, T, 512), torch.bfloat16)
    C = Guarded((1, P, 256, 512), torch.float32)
    n = Guarded((1, P, 256), torch.float32)
    m = Guarded((1, P), torch.float32)
    nb = binding.workspace_size(1, P, T, 256, 512, 64, binding.BF16, variant)
    ws = Guarded((max(nb, 16),), torch.uint8)
    binding.fwd_chunkwise(*[add(d[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")],
                          chunk=64, variant=variant, h=h.t, C_T=C.t, n_T=n.t, m_T=m.t, workspace=ws.t)
    for name, g in (("h", h), ("C_T", C), ("n_T", n), ("m_T", m)):
        g.check(f"prefill {variant} T={T} {name}")
    ws.check(f"prefill {variant} T={T} workspace", finite=False)


def test_prefill_f32_guards():
    w = I.workload("small_f32")
    d = PT.cuda(I.gen_prefill(w, pairs=[(1, 2), (3, 0)], T=99))
    add = lambda t: t.unsqueeze(0)
    h = Guarded((1, 2, 99, 64), torch.float32)
    C = Guarded((1, 2, 64, 64), torch.float32)
    n = Guarded((1, 2, 64), torch.float32)
    m = Guarded((1, 2), torch.float32)
    binding.fwd_chunkwise(*[add(d[k]) for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre", "C0", "n0", "m0")],
                          chunk=32, variant="fused", h=h.t, C_T=C.t, n_T=n.t, m_T=m.t)
    for name, g in (("h", h), ("C_T", C), ("n_T", n), ("m_T", m)):
        g.check(f"prefill f32 {name}")


@pytest.mark.parametrize("split", [True, False])
def test_step_guards(split):
    w = I.workload("decode_bf16")
    Bq = 3
    st = PT.cuda(I.gen_decode_step(w, 0, B=Bq))
    C0, n0, m0 = (x.cuda() for x in I.gen_decode_state(w, B=Bq))
    h = Guarded((Bq, 8, 512), torch.bfloat16)
    C = Guarded((Bq, 8, 256, 512), torch.float32)
    n = Guarded((Bq, 8, 256), torch.float32)
    m = Guarded((Bq, 8), torch.float32)
    ws = None
    if split:
        nb = binding.step_workspace_size(Bq, 8, 256, 512, binding.BF16)
        ws = Guarded((max(nb, 16),), torch.uint8)
    binding.step(*(st[k] for k in ("q", "k", "v", "i_pre", "f_pre", "o_pre")), C0, n0, m0,
                 h=h.t, C_out=C.t, n_out=n.t, m_out=m.t, split=split,
                 workspace=None if ws is None else ws.t)
    for name, g in (("h", h), ("C_out", C), ("n_out", n), ("m_out", m)):
        g.check(f"step split={split} {name}")
    if ws is not None:
        ws.check("step workspace", finite=False)


@pytest.mark.parametrize("name,T,dk,dv", [("small_f32", 70, 64, 64), ("prefill_7b_bf16", 70, 256, 512)])
def test_backward_guards(name, T, dk, dv):
    w = I.workload(name)
    d = PT.cuda(I.gen_prefill(w, pairs=[(0, 1), (1, 0)], T=T))
    io_t = torch.bfloat16 if w.io == "bf16" else torch.float32
    dh = torch.randn((1, 2, T, dv), generator=torch.Generator().manual_seed(5)).to(io_t).cuda()
    add = lambda t: None if t is None else t.unsqueeze(0)
    q, k, v, i_pre, f_pre, o_pre = (add(d[x]) for x in ("q", "k", "v", "i_pre", "f_pre", "o_pre"))
    C0, n0, m0 = add(d["C0"]), add(d["n0"]), add(d["m0"])
    outs = [Guarded(s, torch.float32) for s in ((1, 2, T, dk), (1, 2, T, dk), (1, 2, T, dv), (1, 2, T),
                                                (1, 2, T), (1, 2, T, dv), (1, 2, dk, dv), (1, 2, dk), (1, 2))]
    nb = binding.bwd_workspace_size(1, 2, T, dk, dv, 32, binding.BF16 if w.io == "bf16" else binding.F32)
    ws = Guarded((nb,), torch.uint8)
    p = binding._ptr
    binding._check(binding.lib().mlstm_bwd_chunkwise(
        p(q), p(k), p(v), p(i_pre), p(f_pre), p(o_pre), p(C0), p(n0), p(m0), p(dh),
        *(p(g.t) for g in outs), 1, 2, T, dk, dv, 32, binding._io(q), p(ws.t), nb,
        binding._stream(q.device)))
    for nm, g in zip(("dq", "dk", "dv", "di", "df", "do", "dC0", "dn0", "dm0"), outs):
        g.check(f"backward {name} {nm}")
    ws.check(f"backward {name} workspace", finite=False)


def test_layer_guards():
    w = I.layer_workload("layer_small")
    d = I.gen_layer(w)
    g = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    names = ("x", "W_q", "W_k", "W_v", "W_o", "W_i", "W_f", "b_q", "b_k", "b_v", "b_o", "b_i", "b_f")
    P = w.H * w.B
    h = Guarded((w.H, w.B, w.T, w.d_v), torch.float32)
    C = Guarded((w.H, w.B, w.d_qk, w.d_v), torch.float32)
    n = Guarded((w.H, w.B, w.d_qk), torch.float32)
    m = Guarded((w.H, w.B), torch.float32)
    nb = binding.layer_workspace_size(w.B, w.T, w.d_model, w.H, w.d_qk, w.d_v, w.chunk, binding.F32)
    ws = Guarded((nb,), torch.uint8)
    p = binding._ptr
    binding._check(binding.lib().mlstm_layer_fwd(
        *(p(g[k]) for k in names), p(g["C0"]), p(g["n0"]), p(g["m0"]), p(h.t), p(C.t), p(n.t), p(m.t),
        w.B, w.T, w.d_model, w.H, w.d_qk, w.d_v, w.chunk, binding.F32, p(ws.t), nb,
        binding._stream(g["x"].device)))
    assert P == w.H * w.B
    for name, gd in (("h", h), ("C_T", C), ("n_T", n), ("m_T", m)):
        gd.check(f"layer {name}")
    ws.check("layer workspace", finite=False)


def test_slstm_guards():
    w = I.slstm_workload("slstm_small", T=40)
    d = I.gen_slstm(w)
    g = {k: (v.cuda() if v is not None else None) for k, v in d.items()}
    B_, H, T, dd = w.B, w.H, 40, w.d
    io_t = g["gx"].dtype
    h = Guarded((B_, H, T, dd), io_t)
    st = [Guarded((B_, H, dd), torch.float32) for _ in range(4)]
    binding.slstm_fwd(g["gx"], g["R"], g["c0"], g["n0"], g["m0"], g["h0"], h=h.t,
                      c_T=st[0].t, n_T=st[1].t, m_T=st[2].t, h_T=st[3].t)
    h.check("slstm h")
    for name, gd in zip(("c_T", "n_T", "m_T", "h_T"), st):
        gd.check(f"slstm {name}")
