"""Independent checks ("pins") of the float64 oracle.

Every function here takes an ``oracle.Oracle`` and raises AssertionError when
the oracle disagrees with something the pages or plain mathematics fix.  None
of them reuses the oracle's code: each is a different derivation (the
quadratic, fully parallel form obtained by unrolling the recurrence; the
unstabilized recurrence; causal linear attention; closed forms; a worked
example), written in numpy/scipy float64.

Equations cited are those of the xLSTM note (page "xLSTM", sections "sLSTM"
-- exponential gates and the stabilizer -- and "mLSTM (matrix LSTM)" -- the
matrix memory, normalizer and read-out -- plus its example recurrent step).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TOL = 1e-12  # float64, rounding order differs between the two sides


def relerr(x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    scale = max(float(np.max(np.abs(r))) if r.size else 0.0, 1e-300)
    return float(np.max(np.abs(x - r))) / scale if r.size else 0.0


def _case(rng, T, dk, dv, *, i_mu=0.0, i_sd=2.0, f_mu=1.0, f_sd=2.0, q_scale=1.0,
          state=True, m0_sd=1.0):
    q = rng.standard_normal((T, dk)) * q_scale
    k = rng.standard_normal((T, dk)) / math.sqrt(dk)
    v = rng.standard_normal((T, dv))
    ig = rng.normal(i_mu, i_sd, T)
    fg = -np.logaddexp(0.0, -rng.normal(f_mu, f_sd, T))  # log sigmoid
    og = rng.standard_normal((T, dv)) * 2.0
    if state:
        C0 = rng.standard_normal((dk, dv)) * 0.3
        n0 = rng.standard_normal(dk) * 0.3
        m0 = float(rng.normal(0.0, m0_sd))
    else:
        C0 = np.zeros((dk, dv)); n0 = np.zeros(dk); m0 = 0.0
    return q, k, v, ig, fg, og, C0, n0, m0


def _run(orc, q, k, v, ig, fg, og, C0=None, n0=None, m0=None):
    """One pair through the oracle; returns (h [T,dv], C [dk,dv], n [dk], m)."""
    args = [x[None] for x in (q, k, v, ig, fg, og)]
    if C0 is None:
        h, C, n, m = orc.forward(*args)
    else:
        h, C, n, m = orc.forward(*args, C0[None], n0[None], np.array([m0]))
    return h[0], C[0], n[0], float(m[0])


def quadratic_form(q, k, v, ig, fg, og, C0, n0, m0):
    """The recurrence unrolled into one causal matrix expression.

    With beta_t = sum_{r<=t} f~_r, the unstabilized memory after token t is
    exp(beta_t + m0) C0 + sum_{s<=t} exp(beta_t - beta_s + i~_s) k_s v_s^T, so
    with D_ts = beta_t - beta_s + i~_s (s <= t), gamma_t = beta_t + m0 and
    M_t = max(gamma_t, max_s D_ts) every term is scaled by exp(-M_t)."""
    T = len(ig)
    beta = np.cumsum(fg)
    D = beta[:, None] - beta[None, :] + ig[None, :]
    D = np.where(np.tril(np.ones((T, T), dtype=bool)), D, -np.inf)
    gamma = beta + m0
    M = np.maximum(gamma, D.max(axis=1))
    W = np.exp(D - M[:, None])
    e = np.exp(gamma - M)
    A = W * (q @ k.T)
    num = A @ v + e[:, None] * (q @ C0)
    den = A.sum(axis=1) + e * (q @ n0)
    h = expit(og) * num / np.maximum(np.abs(den), np.exp(-M))[:, None]
    C_T = (W[-1][:, None] * k).T @ v + e[-1] * C0
    n_T = W[-1] @ k + e[-1] * n0
    return h, C_T, n_T, float(M[-1])


def pin_quadratic(orc):
    """P1: sequential oracle == quadratic parallel form (tiny sizes)."""
    rng = np.random.default_rng(101)
    cases = [
        dict(T=1, dk=4, dv=3), dict(T=7, dk=8, dv=5), dict(T=33, dk=16, dv=16),
        dict(T=64, dk=16, dv=8), dict(T=40, dk=5, dv=12, state=False),
        dict(T=50, dk=8, dv=6, q_scale=1e-3),             # normalizer floor binds
        dict(T=30, dk=6, dv=7, i_mu=3.0, f_mu=-1.0),      # stabilizer moves a lot
        dict(T=25, dk=4, dv=9, f_mu=5.0, i_sd=0.1, m0_sd=3.0),
    ]
    for c in cases:
        st = c.pop("state", True)
        args = _case(rng, state=st, **c)
        h, C, n, m = _run(orc, *args)
        hq, Cq, nq, mq = quadratic_form(*args)
        assert relerr(h, hq) <= TOL, ("h", c, relerr(h, hq))
        assert relerr(C, Cq) <= TOL, ("C", c, relerr(C, Cq))
        assert relerr(n, nq) <= TOL, ("n", c, relerr(n, nq))
        assert abs(m - mq) <= TOL * max(1.0, abs(mq)), ("m", c, m, mq)


def unstabilized(q, k, v, ig, fg, og, C0, n0, m0):
    """The note's recurrence taken literally: f = exp(f~), i = exp(i~), no m,
    normalizer floored at one.  The initial stabilized state is first brought
    back to unstabilized variables (times exp(m0))."""
    C = C0 * math.exp(m0)
    n = n0 * math.exp(m0)
    hs = []
    with np.errstate(over="ignore", invalid="ignore"):
        for t in range(len(ig)):
            f, i = math.exp(fg[t]) if fg[t] < 700 else math.inf, \
                math.exp(ig[t]) if ig[t] < 700 else math.inf
            C = f * C + i * np.outer(k[t], v[t])
            n = f * n + i * k[t]
            hs.append(expit(og[t]) * (C.T @ q[t]) / max(abs(n @ q[t]), 1.0))
    return np.array(hs), C, n


def pin_unstabilized(orc):
    """P2: with small exponents the stabilized oracle equals the unstabilized
    recurrence; with a large input gate the unstabilized one overflows while
    the oracle stays finite (and still equals the quadratic form)."""
    rng = np.random.default_rng(202)
    for T, dk, dv in [(20, 6, 5), (12, 3, 8)]:
        args = _case(rng, T, dk, dv, i_sd=0.5, f_mu=2.0, f_sd=1.0, m0_sd=0.5)
        h, C, n, m = _run(orc, *args)
        hu, Cu, nu = unstabilized(*args)
        assert relerr(h, hu) <= 1e-12, ("h", relerr(h, hu))
        assert relerr(C * math.exp(m), Cu) <= 1e-12, ("C", relerr(C * math.exp(m), Cu))
        assert relerr(n * math.exp(m), nu) <= 1e-12
    args = list(_case(rng, 10, 4, 4))
    args[3] = args[3].copy(); args[3][5] = 800.0
    h, C, n, m = _run(orc, *args)
    hu, _, _ = unstabilized(*args)
    assert not np.all(np.isfinite(hu)), "unstabilized form was expected to overflow"
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(C)) and math.isfinite(m)
    hq, Cq, nq, mq = quadratic_form(*args)
    assert relerr(h, hq) <= TOL and relerr(C, Cq) <= TOL and abs(m - mq) <= 1e-9


def pin_linear_attention(orc):
    """P3: i~ = f~ = 0 and a zero start make every gate one and m stay 0, so the
    numerator is unnormalized causal linear attention tril(Q K^T) V and the
    denominator max(|rowsum tril(Q K^T)|, 1)."""
    rng = np.random.default_rng(303)
    for T, dk, dv, qs in [(48, 8, 6, 1.0), (17, 4, 4, 0.05)]:
        q = rng.standard_normal((T, dk)) * qs
        k = rng.standard_normal((T, dk)) * 0.5
        v = rng.standard_normal((T, dv))
        og = rng.standard_normal((T, dv))
        z = np.zeros(T)
        h, C, n, m = _run(orc, q, k, v, z, z, og)
        A = np.tril(q @ k.T)
        lin = A @ v
        den = np.maximum(np.abs(A.sum(axis=1)), 1.0)
        assert m == 0.0
        assert relerr(h / expit(og) * den[:, None], lin) <= 1e-12
        assert relerr(C, k.T @ v) <= 1e-12 and relerr(n, k.sum(axis=0)) <= 1e-12
        if qs < 0.1:  # floor binds on every row: h / sigmoid(o~) is linear attention itself
            assert np.all(np.abs(A.sum(axis=1)) < 1.0)
            assert relerr(h / expit(og), lin) <= 1e-12


def pin_state_carry(orc):
    """P4: running T tokens equals running t0 tokens and continuing from the
    returned state (the state triple is the whole memory of the past)."""
    rng = np.random.default_rng(404)
    q, k, v, ig, fg, og, C0, n0, m0 = _case(rng, 45, 8, 10)
    h, C, n, m = _run(orc, q, k, v, ig, fg, og, C0, n0, m0)
    for t0 in (1, 16, 44):
        h1, C1, n1, m1 = _run(orc, q[:t0], k[:t0], v[:t0], ig[:t0], fg[:t0], og[:t0], C0, n0, m0)
        h2, C2, n2, m2 = _run(orc, q[t0:], k[t0:], v[t0:], ig[t0:], fg[t0:], og[t0:], C1, n1, m1)
        assert relerr(np.concatenate([h1, h2]), h) <= 1e-13
        assert relerr(C2, C) <= 1e-13 and relerr(n2, n) <= 1e-13 and abs(m2 - m) <= 1e-13


def page_step(x, C, n, m):
    """The example recurrent step printed on the note, restated: stabilizer,
    exponential gates, value-first outer-product update of the memory, read-out
    of the memory times the query, normalizer clamped below at one on the
    *stabilized* normalizer, sigmoid output gate.  Only equal to the equations
    when m stays 0."""
    q, k, v, ig, fg, og = x
    m_new = max(fg + m, ig)
    fgate = math.exp(fg + m - m_new)
    igate = math.exp(ig - m_new)
    C = fgate * C + igate * np.outer(v, k)      # d_v x d_qk
    n = fgate * n + igate * k
    h = expit(og) * (C @ q) / max(abs(n @ q), 1.0)
    return h, C, n, m_new


def pin_page_step(orc):
    """P5: with f~ = 0, i~ <= 0 and m0 = 0 the stabilizer never leaves 0, and the
    page's step (which floors the stabilized normalizer at one) must agree with
    the oracle, state orientation included."""
    rng = np.random.default_rng(505)
    T, dk, dv = 24, 6, 9
    q = rng.standard_normal((T, dk)); k = rng.standard_normal((T, dk)) * 0.4
    v = rng.standard_normal((T, dv)); og = rng.standard_normal((T, dv))
    ig = -np.abs(rng.standard_normal(T)); fg = np.zeros(T)
    C = np.zeros((dv, dk)); n = np.zeros(dk); m = 0.0
    hs = []
    for t in range(T):
        h_t, C, n, m = page_step((q[t], k[t], v[t], ig[t], fg[t], og[t]), C, n, m)
        hs.append(h_t)
    h, Co, no, mo = _run(orc, q, k, v, ig, fg, og)
    assert m == 0.0 and mo == 0.0
    assert relerr(h, np.array(hs)) <= 1e-12
    assert relerr(Co, C.T) <= 1e-12 and relerr(no, n) <= 1e-12


def pin_one_token(orc):
    """P6: T = 1 by hand from an arbitrary initial state."""
    rng = np.random.default_rng(606)
    for dk, dv in [(3, 5), (7, 2)]:
        q = rng.standard_normal(dk); k = rng.standard_normal(dk); v = rng.standard_normal(dv)
        og = rng.standard_normal(dv)
        C0 = rng.standard_normal((dk, dv)); n0 = rng.standard_normal(dk)
        for ig, fg, m0 in [(0.3, -0.2, 0.1), (2.5, -1.0, -0.7), (-4.0, 0.5, 1.5)]:
            m1 = max(fg + m0, ig)
            a = math.exp(ig - m1); b = math.exp(fg + m0 - m1)
            num = a * (k @ q) * v + b * (C0.T @ q)
            den = max(abs(a * (k @ q) + b * (n0 @ q)), math.exp(-m1))
            h_ref = expit(og) * num / den
            h, C, n, m = _run(orc, q[None], k[None], v[None], np.array([ig]), np.array([fg]),
                              og[None], C0, n0, m0)
            assert relerr(h[0], h_ref) <= 1e-14
            assert relerr(C, a * np.outer(k, v) + b * C0) <= 1e-14
            assert abs(m - m1) <= 1e-15


def pin_m_closed_form(orc):
    """P7: the stabilizer has the closed form
    m_T = max(m0 + sum_r f~_r, max_s (i~_s + sum_{r>s} f~_r))."""
    rng = np.random.default_rng(707)
    for T in (1, 9, 100):
        q, k, v, ig, fg, og, C0, n0, m0 = _case(rng, T, 3, 2, i_sd=4.0, f_mu=0.0, f_sd=3.0)
        fg = fg + rng.normal(0, 0.5, T)  # some positive log forget gates too
        _, _, _, m = _run(orc, q, k, v, ig, fg, og, C0, n0, m0)
        tail = np.concatenate([np.cumsum(fg[::-1])[::-1][1:], [0.0]])  # sum_{r>s}
        m_ref = max(m0 + fg.sum(), float(np.max(ig + tail)))
        assert abs(m - m_ref) <= 1e-12 * max(1.0, abs(m_ref)), (m, m_ref)


def pin_hand_example(orc):
    """The two-token example worked by hand in tests/golden/hand_T2.json."""
    with open(os.path.join(GOLDEN, "hand_T2.json")) as f:
        g = json.load(f)
    val = {"0": 0.0, "ln2": math.log(2.0), "-ln2": -math.log(2.0),
           "ln3": math.log(3.0), "-ln3": -math.log(3.0)}
    q = np.array(g["q"]); k = np.array(g["k"]); v = np.array(g["v"])
    ig = np.array([val[s] for s in g["i_pre"]]); fg = np.array([val[s] for s in g["f_pre"]])
    og = np.array([[val[s] for s in row] for row in g["o_pre"]])
    h, C, n, m = _run(orc, q, k, v, ig, fg, og)
    assert np.max(np.abs(h - np.array(g["h"]))) <= 1e-14, h
    assert np.max(np.abs(C - np.array(g["C_T"]))) <= 1e-14, C
    assert np.max(np.abs(n - np.array(g["n_T"]))) <= 1e-14
    assert abs(m - g["m_T"]) <= 1e-15


def pin_extreme_output_gate(orc):
    """The output gate saturates to exactly 0 and 1 without NaN for |o~| huge."""
    T, dk, dv = 3, 2, 2
    q = np.ones((T, dk)); k = np.ones((T, dk)); v = np.ones((T, dv))
    og = np.array([[800.0, -800.0]] * T)
    h, _, _, _ = _run(orc, q, k, v, np.zeros(T), np.zeros(T), og)
    assert np.all(np.isfinite(h)) and np.all(h[:, 1] == 0.0) and np.all(h[:, 0] > 0)


ALL_PINS = [pin_quadratic, pin_unstabilized, pin_linear_attention, pin_state_carry,
            pin_page_step, pin_one_token, pin_m_closed_form, pin_hand_example,
            pin_extreme_output_gate]
