"""Pins of the oracle's backward pass (CPU only).

The gradients are checked against central finite differences of the forward
oracle, itself pinned in test_oracle_pins.py: the loss is sum(dh * h), each
input element is moved by +-eps and the difference quotient is compared with
the analytic gradient.  The cases avoid the kinks of the read-out (the floor
of the normalizer, and n.q = 0), where the derivative is one-sided: a guard
draws the inputs again when a token sits near one.  Two identities that the
oracle does not use are checked as well: the input-gate gradient is k . dk,
and the forget-gate gradient is the reverse cumulative sum of q . dq - k . dk.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")

EPS = 1e-6
RTOL = 1e-6


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _near_kink(q, k, v, ig, fg, C0, n0, m0):
    """True when some token's |n.q| is within 1e-3 (relative) of the floor
    exp(-m) or of zero (plain float64 recurrence, a guard only)."""
    P, T, dk = q.shape
    for p in range(P):
        n = np.zeros(dk) if n0 is None else n0[p].copy()
        m = 0.0 if m0 is None else m0[p]
        for t in range(T):
            mn = max(fg[p, t] + m, ig[p, t])
            n = np.exp(fg[p, t] + m - mn) * n + np.exp(ig[p, t] - mn) * k[p, t]
            m = mn
            d = abs(n @ q[p, t])
            fl = np.exp(-m)
            if abs(d - fl) < 1e-3 * fl or d < 1e-9:
                return True
    return False


def _case(seed, P=2, T=6, dk=3, dv=4, state=False, qscale=1.0, spikes=False):
    rng = np.random.default_rng(seed)
    while True:
        q = rng.normal(size=(P, T, dk)) * qscale
        k = rng.normal(size=(P, T, dk)) / np.sqrt(dk)
        v = rng.normal(size=(P, T, dv))
        ig = rng.normal(-1.0, 1.0, size=(P, T))
        if spikes:
            ig[:, T // 3] = 30.0
            ig[:, 2 * T // 3] = -30.0
        fg = -np.log1p(np.exp(-rng.normal(2.0, 1.0, size=(P, T))))
        og = rng.normal(size=(P, T, dv))
        dh = rng.normal(size=(P, T, dv))
        C0 = n0 = m0 = None
        if state:
            C0 = rng.normal(0.0, 0.5, size=(P, dk, dv))
            n0 = rng.normal(0.0, 0.5, size=(P, dk))
            m0 = rng.uniform(-1.0, 1.0, size=P)
        if not _near_kink(q, k, v, ig, fg, C0, n0, m0):
            return dict(q=q, k=k, v=v, i_pre=ig, f_pre=fg, o_pre=og, C0=C0, n0=n0, m0=m0), dh


def _loss(inp, dh):
    h = oracle.forward(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], inp["o_pre"],
                       inp["C0"], inp["n0"], inp["m0"])[0]
    return float((h * dh).sum())


def _fd(inp, dh, name):
    x = inp[name]
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        keep = x[idx]
        x[idx] = keep + EPS
        lp = _loss(inp, dh)
        x[idx] = keep - EPS
        lm = _loss(inp, dh)
        x[idx] = keep
        g[idx] = (lp - lm) / (2 * EPS)
    return g


NAMES = ["q", "k", "v", "i_pre", "f_pre", "o_pre"]
STATE = ["C0", "n0", "m0"]


@pytest.mark.parametrize("kw", [
    dict(seed=1),
    dict(seed=2, state=True),
    dict(seed=3, qscale=0.5, state=True),  # smaller q: the floor is active for most tokens
    dict(seed=4, spikes=True, state=True, T=9),  # input gates of +-30: the stabilizer moves
    dict(seed=5, T=1, state=True),
])
def test_backward_matches_finite_differences(kw):
    inp, dh = _case(**kw)
    got = oracle.backward(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], inp["o_pre"], dh,
                          inp["C0"], inp["n0"], inp["m0"])
    names = NAMES + (STATE if kw.get("state") else [])
    for name in names:
        ref = _fd(inp, dh, name)
        g = got[(NAMES + STATE).index(name)]
        err = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-12)
        assert err <= RTOL, (kw, name, err)


def test_floor_case_has_floor_active():
    """The smaller-q case above exercises both branches of the read-out's
    denominator (a guard on the case itself): some tokens have |n.q| below
    the floor exp(-m), others above it."""
    inp, _ = _case(seed=3, qscale=0.5, state=True)
    q, k, ig, fg = inp["q"], inp["k"], inp["i_pre"], inp["f_pre"]
    n0, m0 = inp["n0"], inp["m0"]
    below = above = 0
    for p in range(q.shape[0]):
        n, m = n0[p].copy(), m0[p]
        for t in range(q.shape[1]):
            mn = max(fg[p, t] + m, ig[p, t])
            n = np.exp(fg[p, t] + m - mn) * n + np.exp(ig[p, t] - mn) * k[p, t]
            m = mn
            if abs(n @ q[p, t]) < np.exp(-m):
                below += 1
            else:
                above += 1
    assert below > 0 and above > 0


@pytest.mark.parametrize("seed", [11, 12])
def test_gate_gradient_identities(seed):
    """di = k . dk and df_t = sum_{s >= t} (q_s . dq_s - k_s . dk_s): the
    oracle computes both gates' gradients from their own definitions
    (<dC*, C_{t-1}> terms), so these are independent cross-checks."""
    inp, dh = _case(seed, P=3, T=20, dk=5, dv=6, state=True)
    dq, dk, dv, di, df, do, dC0, dn0, dm0 = oracle.backward(
        inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], inp["o_pre"], dh,
        inp["C0"], inp["n0"], inp["m0"])
    q, k = inp["q"], inp["k"]
    np.testing.assert_allclose(di, (k * dk).sum(-1), rtol=1e-10, atol=1e-12)
    x = (q * dq).sum(-1) - (k * dk).sum(-1)
    rev = np.cumsum(x[:, ::-1], axis=1)[:, ::-1]
    np.testing.assert_allclose(df, rev, rtol=1e-9, atol=1e-11)


def test_output_gate_gradient_closed_form():
    """do = dh * h * (1 - sigmoid(o~)): h / sigmoid(o~) does not depend on o~."""
    inp, dh = _case(21, state=True)
    h = oracle.forward(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], inp["o_pre"],
                       inp["C0"], inp["n0"], inp["m0"])[0]
    do = oracle.backward(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], inp["o_pre"], dh,
                         inp["C0"], inp["n0"], inp["m0"])[5]
    np.testing.assert_allclose(do, dh * h * (1.0 - _sigmoid(inp["o_pre"])), rtol=1e-10, atol=1e-14)


# ---- the pins catch plausible mistakes in the backward (planted in a copy
# of the source, on the CPU; the real oracle is never modified)

BWD_MUTANTS = [
    ("beta_dropped", "beta = -(nq[t] > 0.0 ? 1.0 : -1.0) * an / den[t];", "beta = 0.0;"),
    ("beta_sign", "beta = -(nq[t] > 0.0 ? 1.0 : -1.0) * an / den[t];",
     "beta = (nq[t] > 0.0 ? 1.0 : -1.0) * an / den[t];"),
    ("decay_index", "dCs[r * dv + b] = qt[r] * a[b] + fpv[t + 1] * dCs[r * dv + b];",
     "dCs[r * dv + b] = qt[r] * a[b] + fpv[t] * dCs[r * dv + b];"),
    ("dv_input_gate_dropped", "dvv[t * dv + b] = ipv[t] * s;", "dvv[t * dv + b] = s;"),
    ("dq_normalizer_dropped", "dq[t * dk + r] = cq + n[r] * beta;", "dq[t * dk + r] = cq;"),
    ("df_current_state", "sdf += dCs[r * dv + b] * Cp[r * dv + b];", "sdf += dCs[r * dv + b] * C[r * dv + b];"),
    ("do_sigmoid_derivative", "dog[t * dv + b] = g[b] * nt[b] / den[t] * sg * (1.0 - sg);",
     "dog[t * dv + b] = g[b] * nt[b] / den[t] * sg;"),
    ("dm0_normalizer_dropped", "s0 += g1 * ns[r];", "s0 += 0.0 * g1 * ns[r];"),
    ("dk_normalizer_dropped", "dkk[t * dk + r] = ipv[t] * (dcv + dns[r]);", "dkk[t * dk + r] = ipv[t] * dcv;"),
]


def _pin_backward(orc):
    """Finite differences of orc's own forward against orc's backward."""
    for kw in (dict(seed=31, state=True), dict(seed=32, state=True, qscale=0.5)):
        inp, dh = _case(**kw)
        got = orc.backward(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], inp["o_pre"], dh,
                           inp["C0"], inp["n0"], inp["m0"])

        def loss():
            h = orc.forward(inp["q"], inp["k"], inp["v"], inp["i_pre"], inp["f_pre"], inp["o_pre"],
                            inp["C0"], inp["n0"], inp["m0"])[0]
            return float((h * dh).sum())

        for j, name in enumerate(NAMES + STATE):
            x = inp[name]
            ref = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                keep = x[idx]
                x[idx] = keep + EPS
                lp = loss()
                x[idx] = keep - EPS
                lm = loss()
                x[idx] = keep
                ref[idx] = (lp - lm) / (2 * EPS)
            err = np.abs(got[j] - ref).max() / max(np.abs(ref).max(), 1e-12)
            assert err <= RTOL, (name, err)


@pytest.mark.parametrize("name,old,new", BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_backward_mutant_is_caught(tmp_path, name, old, new):
    import os
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = os.path.join(tmp_path, "mutant.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(src=mpath, out=os.path.join(tmp_path, f"libmut_{name}.so"),
                       extra_flags=("-Wno-error", "-w"))
    with pytest.raises(AssertionError):
        _pin_backward(oracle.Oracle(lib))


def test_backward_pin_passes_on_the_oracle():
    _pin_backward(oracle.load())
