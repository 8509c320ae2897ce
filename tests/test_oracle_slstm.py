"""Pins of the sLSTM oracle (oracle/slstm_ref.c), on the CPU.

Facts fixed independently of its code:
- without memory mixing (R = 0) and from the zero state, c_t / n_t is the
  average of tanh(z~_s) over s <= t with weights exp(i~_s + sum_{r=s+1..t}
  f~_r): a closed form evaluated here by a stable softmax, not a recurrence;
  m_T is the mLSTM's closed form per cell;
- the stabilizer cancels: the literal recurrence (f = e^{f~}, i = e^{i~},
  no m) gives the same h wherever it does not overflow;
- memory mixing runs from h_{t-1} along the rows of R: with a single entry
  R[g][0][1] cell 0 hears cell 1 one step later, and cell 1 never hears 0;
- a state carried across two calls equals one call.
Planted mistakes in copies of the C source must each fail one of them."""
import os

import numpy as np
import pytest

from oracle import slstm as S

B, H, T, D = 2, 3, 29, 5


def draw(seed, B=B, H=H, T=T, D=D, rscale=0.3, state=False):
    rng = np.random.default_rng(seed)
    gx = rng.normal(0.0, 1.0, (B, H, T, 4, D))
    gx[..., 1, :] += -0.5            # input gates
    gx[..., 2, :] = rng.normal(1.0, 0.5, (B, H, T, D))   # forget pre-activations (log gates)
    R = rng.normal(0.0, rscale, (H, 4, D, D))
    st = None
    if state:
        st = (rng.normal(0, 0.5, (B, H, D)), np.abs(rng.normal(1.0, 0.2, (B, H, D))),
              rng.uniform(-1, 1, (B, H, D)), rng.normal(0, 0.5, (B, H, D)))
    return gx, R, st


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def pin_weighted_average(fwd):
    gx, R, _ = draw(1)
    R[:] = 0.0
    gx[..., 2, :] = np.random.default_rng(5).normal(-0.3, 0.4, (B, H, T, D))  # either sign
    h, (c, n, m, hT) = fwd(gx, R)
    z, i, f, o = (gx[..., g, :] for g in range(4))          # [B, H, T, D]
    for t in range(T):
        # log weights of tokens s <= t: i_s + sum_{r=s+1..t} f_r
        tail = np.cumsum(f[:, :, t::-1], axis=2)[:, :, ::-1] - f[:, :, :t + 1]
        lw = i[:, :, :t + 1] + tail
        w = np.exp(lw - lw.max(axis=2, keepdims=True))
        avg = (w * np.tanh(z[:, :, :t + 1])).sum(2) / w.sum(2)
        np.testing.assert_allclose(h[:, :, t], sigmoid(o[:, :, t]) * avg, rtol=1e-11, atol=1e-13)
    tail = np.cumsum(f[:, :, ::-1], axis=2)[:, :, ::-1] - f
    mref = np.maximum(f.sum(2), (i + tail).max(2))
    np.testing.assert_allclose(m, mref, rtol=0, atol=1e-12)
    lw = i + tail
    np.testing.assert_allclose(n, np.exp(lw - mref[:, :, None, :]).sum(2), rtol=1e-11)
    np.testing.assert_allclose(c, (np.exp(lw - mref[:, :, None, :]) * np.tanh(z)).sum(2), rtol=1e-10,
                               atol=1e-13)


def literal(gx, R, state=None):
    """The recurrence taken literally: exponential gates, no stabilizer."""
    Bn, Hn, Tn, _, Dn = gx.shape
    h = np.zeros((Bn, Hn, Tn, Dn))
    for b in range(Bn):
        for hh in range(Hn):
            c = np.zeros(Dn); n = np.zeros(Dn); hp = np.zeros(Dn)
            if state is not None:
                c0, n0, m0, h0 = (x[b, hh] for x in state)
                c, n, hp = c0 * np.exp(m0), n0 * np.exp(m0), h0.copy()
            for t in range(Tn):
                pre = gx[b, hh, t] + np.einsum("gjk,k->gj", R[hh], hp)
                c = np.exp(pre[2]) * c + np.exp(pre[1]) * np.tanh(pre[0])
                n = np.exp(pre[2]) * n + np.exp(pre[1])
                hp = sigmoid(pre[3]) * c / n
                h[b, hh, t] = hp
    return h


def pin_literal(fwd):
    for state in (False, True):
        gx, R, st = draw(2, state=state)
        h, _ = fwd(gx, R, *(st or ()))
        np.testing.assert_allclose(h, literal(gx, R, st), rtol=1e-10, atol=1e-12)


def pin_mixing_direction(fwd):
    gx, R, _ = draw(3, B=1, H=1, T=12, D=3)
    R[:] = 0.0
    R[0, :, 0, 1] = [0.9, -0.7, 0.5, 0.8]      # cell 0 reads cell 1, through every gate
    h, _ = fwd(gx, R)
    # perturb cell 1 at token 5: cell 1 changes from 5 on, cell 0 from 6 on
    g2 = gx.copy(); g2[0, 0, 5, 0, 1] += 0.7
    h2, _ = fwd(g2, R)
    d0 = np.abs(h2[0, 0, :, 0] - h[0, 0, :, 0])
    d1 = np.abs(h2[0, 0, :, 1] - h[0, 0, :, 1])
    assert np.all(d1[:5] == 0) and d1[5] > 0
    assert np.all(d0[:6] == 0) and d0[6] > 0
    # perturb cell 0: cell 1 never moves
    g3 = gx.copy(); g3[0, 0, 2, 0, 0] += 0.7
    h3, _ = fwd(g3, R)
    assert np.all(h3[0, 0, :, 1] == h[0, 0, :, 1])
    assert np.all(h3[0, 0, :2, 0] == h[0, 0, :2, 0]) and h3[0, 0, 2, 0] != h[0, 0, 2, 0]
    # cell 2 is isolated
    assert np.all(h3[0, 0, :, 2] == h[0, 0, :, 2]) and np.all(h2[0, 0, :, 2] == h[0, 0, :, 2])


def pin_state_carry(fwd):
    gx, R, st = draw(4, state=True)
    h, (c, n, m, hT) = fwd(gx, R, *st)
    h1, s1 = fwd(gx[:, :, :11], R, *st)
    h2, (c2, n2, m2, hT2) = fwd(gx[:, :, 11:], R, *s1)
    np.testing.assert_allclose(np.concatenate([h1, h2], axis=2), h, rtol=1e-13, atol=1e-15)
    for x, y in ((c2, c), (n2, n), (m2, m), (hT2, hT)):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(hT, h[:, :, -1])


PINS = (pin_weighted_average, pin_literal, pin_mixing_direction, pin_state_carry)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(S.forward)


def test_zero_state_equals_explicit_zero_state():
    gx, R, _ = draw(6)
    z = np.zeros((B, H, D))
    h1, s1 = S.forward(gx, R)
    h2, s2 = S.forward(gx, R, z, z, z, z)
    np.testing.assert_array_equal(h1, h2)


SLSTM_MUTANTS = [
    ("no_tanh", "const double zt = tanh(pre[j]);", "const double zt = pre[j];"),
    ("gates_swapped", "const double it = pre[d + j], ft = pre[2 * d + j]",
     "const double it = pre[2 * d + j], ft = pre[d + j]"),
    ("R_transposed", "s += row[k] * hp[k];", "s += ((void)row, R[((size_t)gi * d + k) * d + j]) * hp[k];"),
    ("stale_mixing_state", "        memcpy(hp, ht, (size_t)d * sizeof(double));\n    }",
     "        if (t % 2) memcpy(hp, ht, (size_t)d * sizeof(double));\n    }"),
    ("normalizer_without_input_gate", "n[j] = fp * n[j] + ip;", "n[j] = fp * n[j] + 1.0;"),
    ("stabilizer_not_carried", "m[j] = mnew;", "m[j] = 0.0;"),
    ("no_output_gate", "ht[j] = sigmoid(ot) * c[j] / n[j];", "ht[j] = 2.0 * sigmoid(0.0) * ((void)ot, c[j] / n[j]);"),
    ("forget_not_rescaled", "const double fp = exp(ft + m[j] - mnew);", "const double fp = exp(ft - mnew);"),
]


@pytest.mark.parametrize("name,old,new", SLSTM_MUTANTS, ids=[m[0] for m in SLSTM_MUTANTS])
def test_slstm_mutant_is_caught(tmp_path, name, old, new):
    with open(S.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, name
    src = src.replace(old, new)
    mpath = os.path.join(tmp_path, f"mut_{name}.c")
    with open(mpath, "w") as f:
        f.write(src)
    lib = S.build(src=mpath, out=os.path.join(tmp_path, f"libmut_{name}.so"))
    fwd = S.SlstmOracle(lib).forward
    caught = False
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught = True
    assert caught, f"mutant {name} passed every pin"
