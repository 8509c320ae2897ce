"""Pins of the layer oracle (oracle/layer.py), on the CPU.

Two facts fixed independently of its code:
- with selection weights (each head's projections pick their own columns of
  x) the layer is the cell on those columns plus the biases, cells ordered
  head-major: checked against the cell oracle, itself pinned in
  test_oracle_pins.py;
- one token from the zero state has a closed form: the memory is i' k v^T, so
  h = sigmoid(o) * v (k.q) i' / max(i' |k.q|, e^{-m}) with m = max(f~, i~)
  and i' = e^{i~ - m}.
Planted mistakes (a dropped bias, swapped projections or gates, another cell
order, a wrong sign) must each fail one of them."""
import numpy as np
import pytest

import oracle
from oracle import layer as L

H, B, T, DK, DV = 2, 3, 37, 4, 6


def selection_case(seed=0):
    """Weights that copy distinct slices of x: head h's q reads columns
    [off, off + dk) etc.  Returns the layer's arguments and the cell inputs
    they must produce."""
    rng = np.random.default_rng(seed)
    widths = [("q", DK), ("k", DK), ("v", DV), ("o", DV), ("i", 1), ("f", 1)]
    per_head = sum(w for _, w in widths)
    D = H * per_head + 3                       # three unused columns
    x = rng.normal(0.0, 1.0, (B, T, D))
    W = {n: np.zeros((H, w, D)) for n, w in widths}
    bias = {n: rng.normal(0.0, 0.5, (H, w)) for n, w in widths}
    cols = {}
    off = 0
    for h in range(H):
        for n, w in widths:
            W[n][h, np.arange(w), off + np.arange(w)] = 1.0
            cols[(n, h)] = slice(off, off + w)
            off += w
    bias["f"] += 3.0                            # forget gates near one
    args = (x, W["q"], W["k"], W["v"], W["o"], W["i"][:, 0], W["f"][:, 0],
            bias["q"], bias["k"], bias["v"], bias["o"], bias["i"][:, 0], bias["f"][:, 0])
    cell = {}
    for n, _ in widths:
        per = [x[:, :, cols[(n, h)]] + bias[n][h] for h in range(H)]   # [B, T, w] each
        y = np.stack(per)                                                # [H, B, T, w]
        cell[n] = y.reshape(H * B, T, -1)
    cell["i"] = cell["i"][..., 0]
    cell["f"] = cell["f"][..., 0]
    return args, cell


def pin_selection(layer_forward):
    args, c = selection_case()
    rng = np.random.default_rng(7)
    C0 = rng.normal(0.0, 0.1, (H, B, DK, DV))
    n0 = rng.normal(0.0, 0.1, (H, B, DK))
    m0 = rng.uniform(-1.0, 1.0, (H, B))
    h, C, n, m = layer_forward(*args, C0, n0, m0)
    hr, Cr, nr, mr = oracle.forward(c["q"], c["k"], c["v"], c["i"], c["f"], c["o"],
                                    C0.reshape(H * B, DK, DV), n0.reshape(H * B, DK),
                                    m0.reshape(H * B))
    np.testing.assert_allclose(h.reshape(H * B, T, DV), hr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(C.reshape(H * B, DK, DV), Cr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(n.reshape(H * B, DK), nr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(m.reshape(H * B), mr, rtol=1e-12, atol=1e-12)


def pin_single_token(layer_forward, seed=3):
    rng = np.random.default_rng(seed)
    D = 11
    x = rng.normal(0.0, 1.0, (B, 1, D))
    Wq, Wk = rng.normal(0, 0.5, (H, DK, D)), rng.normal(0, 0.5, (H, DK, D))
    Wv, Wo = rng.normal(0, 0.5, (H, DV, D)), rng.normal(0, 0.5, (H, DV, D))
    Wi, Wf = rng.normal(0, 0.5, (H, D)), rng.normal(0, 0.5, (H, D))
    bq, bk = rng.normal(0, 0.5, (H, DK)), rng.normal(0, 0.5, (H, DK))
    bv, bo = rng.normal(0, 0.5, (H, DV)), rng.normal(0, 0.5, (H, DV))
    bi, bf = rng.normal(0, 0.5, H), rng.normal(0, 0.5, H)
    h, C, n, m = layer_forward(x, Wq, Wk, Wv, Wo, Wi, Wf, bq, bk, bv, bo, bi, bf)
    for hh in range(H):
        for b in range(B):
            xt = x[b, 0]
            q, k = Wq[hh] @ xt + bq[hh], Wk[hh] @ xt + bk[hh]
            v, o = Wv[hh] @ xt + bv[hh], Wo[hh] @ xt + bo[hh]
            ig, fg = Wi[hh] @ xt + bi[hh], Wf[hh] @ xt + bf[hh]
            mt = max(fg, ig)
            ip = np.exp(ig - mt)
            kq = k @ q
            expect = v * kq * ip / max(ip * abs(kq), np.exp(-mt)) / (1.0 + np.exp(-o))
            np.testing.assert_allclose(h[hh, b, 0], expect, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(C[hh, b], ip * np.outer(k, v), rtol=1e-12, atol=1e-15)
            np.testing.assert_allclose(n[hh, b], ip * k, rtol=1e-12, atol=1e-15)
            assert m[hh, b] == pytest.approx(mt, abs=1e-14)


def test_selection_weights_reduce_to_the_cell():
    pin_selection(L.layer_forward)


def test_single_token_closed_form():
    pin_single_token(L.layer_forward)


def test_bf16_rounding():
    """round_bf16 against torch's own bfloat16 cast on float32 values (one
    rounding either way there), on ties, and on its defining properties."""
    import torch
    rng = np.random.default_rng(11)
    a = rng.normal(0.0, 1.0, 100000).astype(np.float32).astype(np.float64) * 2.0 ** rng.integers(-20, 20, 100000)
    t = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(L.round_bf16(a), t)
    # ties go to the even neighbour: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert L.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert L.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert L.round_bf16(-(1.0 + 2.0 ** -8)) == -1.0
    # idempotent, and within half an ulp (2^-9 relative) of the input
    r = L.round_bf16(a)
    np.testing.assert_array_equal(L.round_bf16(r), r)
    assert np.all(np.abs(r - a) <= np.abs(a) * 2.0 ** -8)


def test_bf16_io_rounds_the_cell_inputs():
    """With bf16 I/O the layer equals the cell on the rounded selection
    outputs."""
    args, c = selection_case()
    h, C, n, m = L.layer_forward(*args, io="bf16")
    rd = {k: (L.round_bf16(c[k]) if k in "qkvo" else c[k]) for k in c}
    hr, Cr, nr, mr = oracle.forward(rd["q"], rd["k"], rd["v"], rd["i"], rd["f"], rd["o"])
    np.testing.assert_allclose(h.reshape(H * B, T, DV), hr, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        L.layer_forward(*args, io="f16")


def test_shapes_and_dtypes_of_projections():
    args, _ = selection_case()
    q, k, v, o, i, f = L.projections(*args)
    assert q.shape == (H, B, T, DK) and v.shape == (H, B, T, DV)
    assert i.shape == (H, B, T) and f.shape == (H, B, T)
    assert all(a.dtype == np.float64 for a in (q, k, v, o, i, f))


LAYER_MUTANTS = [
    ("bias_dropped", "y = np.stack([x @ W[h].T + b[h] for h in range(W.shape[0])])",
     "y = np.stack([x @ W[h].T for h in range(W.shape[0])])"),
    ("gates_swapped", "for W, b in ((W_i, b_i), (W_f, b_f)):", "for W, b in ((W_f, b_f), (W_i, b_i)):"),
    ("q_k_swapped", "for W, b in ((W_q, b_q), (W_k, b_k), (W_v, b_v), (W_o, b_o)):",
     "for W, b in ((W_k, b_k), (W_q, b_q), (W_v, b_v), (W_o, b_o)):"),
    ("v_o_swapped", "for W, b in ((W_q, b_q), (W_k, b_k), (W_v, b_v), (W_o, b_o)):",
     "for W, b in ((W_q, b_q), (W_k, b_k), (W_o, b_o), (W_v, b_v)):"),
    ("batch_major_cells", "        out.append(y)", "        out.append(np.ascontiguousarray(y.swapaxes(0, 1)))"),
    ("gate_bias_sign", "out.append(np.stack([x @ W[h] + b[h] for h in range(W.shape[0])]))",
     "out.append(np.stack([x @ W[h] - b[h] for h in range(W.shape[0])]))"),
    ("gate_bias_one_head", "out.append(np.stack([x @ W[h] + b[h] for h in range(W.shape[0])]))",
     "out.append(np.stack([x @ W[h] + b[0] for h in range(W.shape[0])]))"),
]


@pytest.mark.parametrize("name,old,new", LAYER_MUTANTS, ids=[m[0] for m in LAYER_MUTANTS])
def test_layer_mutant_is_caught(name, old, new):
    with open(L.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, name
    src = src.replace(old, new).replace("from . import forward as cell_forward",
                                        "from oracle import forward as cell_forward")
    ns = {"__name__": f"layer_mutant_{name}"}
    exec(compile(src, f"<mutant {name}>", "exec"), ns)
    caught = False
    for pin in (pin_selection, pin_single_token):
        try:
            pin(ns["layer_forward"])
        except (AssertionError, ValueError):
            caught = True
    assert caught, f"mutant {name} passed every pin"
