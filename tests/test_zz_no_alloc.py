"""mlstm_step_noalloc (the step for callers that cannot allocate device
memory) against mlstm_step given a workspace: both run the same row-split
kernels, the first in the library's fixed per-device scratch, so every output
must be bitwise equal.  Calls follow one another on the same device, the
later ones smaller, so a call that read partial results left in the shared
scratch by an earlier, larger call would show up as a mismatch."""
import pytest
import torch

import oracle
from tests import parity as PT
from xlstm_mlstm_matrix_amd import binding, inputs as I

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


def both(st, state):
    """(h, C, n, m) of mlstm_step with a fresh workspace and of
    mlstm_step_noalloc, from the same inputs and initial state (not updated
    in place, so both read the same state)."""
    x = [st[k] for k in NAMES]
    ref = binding.step(*x, *state, inplace=False, split=True)
    got = binding.step_noalloc(*x, *state, inplace=False)
    torch.cuda.synchronize()
    return ref, got


def assert_same(ref, got, what):
    for name, a, b in zip(("h", "C", "n", "m"), ref, got):
        assert a.shape == b.shape and torch.equal(a, b), f"{what}: {name} differs"


def decode_inputs(io, B, dk, dv, state=True):
    w = I.workload("decode_bf16", io=io, d_qk=dk, d_v=dv)
    st = PT.cuda(I.gen_decode_step(w, 0, B=B))
    C0 = n0 = m0 = None
    if state:
        C0, n0, m0 = (t.cuda() for t in I.gen_decode_state(w, B=B))
    return st, (C0, n0, m0)


def test_two_calls_in_a_row_second_smaller():
    """Full decode batch (256 x 8 cells of 256 x 512: 16.9 MB of partials),
    then 24 x 8 cells: the second call must not see the first call's partials."""
    for B in (256, 24):
        print(f"noalloc bf16 B={B} 256x512", flush=True)
        st, state = decode_inputs("bf16", B, 256, 512)
        ref, got = both(st, state)
        assert_same(ref, got, f"B={B}")


def test_small_against_oracle_then_again():
    """f32 I/O, zero initial state, a ragged last row block (208 rows in
    blocks of 64): the no-allocation step equals the oracle to the step's
    tolerance, and a second, smaller call equals mlstm_step."""
    for B in (6, 2):
        print(f"noalloc f32 B={B} 208x512 zero state", flush=True)
        st, state = decode_inputs("f32", B, 208, 512, state=False)
        ref, got = both(st, state)
        assert_same(ref, got, f"f32 B={B}")
        P = B * 8
        r = oracle.forward(*(st[k].cpu().reshape(P, 1, *st[k].shape[2:]) for k in NAMES))
        flat = lambda t: t.reshape(P, *t.shape[2:])
        h, C, n, m = got
        PT.compare_fwd((flat(h).unsqueeze(1), flat(C), flat(n), flat(m)), r, "f32", f"oracle B={B}")


def test_shape_without_split_uses_no_scratch():
    """64 x 64 cells have one row block: the one-workgroup kernel runs, as
    for mlstm_step, whatever the scratch holds."""
    print("noalloc bf16 B=16 64x64", flush=True)
    st, state = decode_inputs("bf16", 16, 64, 64)
    ref, got = both(st, state)
    assert_same(ref, got, "64x64")


def test_largest_batch_that_fits():
    """4064 cells of 256 x 512 (33 552 384 bytes of partials in the
    33 554 432-byte scratch), then 4065 cells, which do not fit, are refused
    with MLSTM_ERR_SCRATCH before any device work."""
    print("noalloc bf16 B=508 H=8 256x512 (largest)", flush=True)
    g = torch.Generator(device="cuda").manual_seed(17)
    B, H, dk, dv = 508, 8, 256, 512
    r = lambda *s: torch.randn(*s, device="cuda", generator=g)
    st = {"q": r(B, H, dk).bfloat16(), "k": (r(B, H, dk) / 16).bfloat16(), "v": r(B, H, dv).bfloat16(),
          "i_pre": r(B, H), "f_pre": torch.nn.functional.logsigmoid(r(B, H) + 3),
          "o_pre": r(B, H, dv).bfloat16()}
    state = (r(B, H, dk, dv) * 0.05, r(B, H, dk) * 0.05, r(B, H))
    ref, got = both(st, state)
    assert_same(ref, got, "B=508 H=8")
    del ref, got, state
    x = {k: t[:1].expand(4065, *t.shape[1:])[:, :1].contiguous() for k, t in st.items()}
    with pytest.raises(binding.MlstmError) as e:
        binding.step_noalloc(*(x[k] for k in NAMES))
    assert e.value.status == 10
