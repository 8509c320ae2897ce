"""The float64 oracle against its independent pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIB)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_pairs_are_independent_and_threads_do_not_matter(orc):
    """Several pairs in one call == each pair alone; thread count is irrelevant."""
    rng = np.random.default_rng(9)
    P, T, dk, dv = 5, 19, 6, 7
    q = rng.standard_normal((P, T, dk)); k = rng.standard_normal((P, T, dk))
    v = rng.standard_normal((P, T, dv)); o = rng.standard_normal((P, T, dv))
    i = rng.normal(0, 2, (P, T)); f = -np.logaddexp(0, -rng.normal(1, 2, (P, T)))
    C0 = rng.standard_normal((P, dk, dv)); n0 = rng.standard_normal((P, dk)); m0 = rng.standard_normal(P)
    full = orc.forward(q, k, v, i, f, o, C0, n0, m0, threads=3)
    one = orc.forward(q, k, v, i, f, o, C0, n0, m0, threads=1)
    for a, b in zip(full, one):
        assert np.array_equal(a, b)
    for p in range(P):
        s = orc.forward(q[p:p+1], k[p:p+1], v[p:p+1], i[p:p+1], f[p:p+1], o[p:p+1],
                        C0[p:p+1], n0[p:p+1], m0[p:p+1])
        for a, b in zip(full, s):
            assert np.array_equal(a[p], b[0])


def test_zero_state_equals_explicit_zero(orc):
    rng = np.random.default_rng(10)
    P, T, dk, dv = 2, 11, 4, 3
    args = [rng.standard_normal((P, T, dk)), rng.standard_normal((P, T, dk)),
            rng.standard_normal((P, T, dv)), rng.normal(0, 1, (P, T)),
            -np.logaddexp(0, -rng.normal(2, 1, (P, T))), rng.standard_normal((P, T, dv))]
    a = orc.forward(*args)
    b = orc.forward(*args, np.zeros((P, dk, dv)), np.zeros((P, dk)), np.zeros(P))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_partial_state_rejected(orc):
    z = np.zeros((1, 2, 2))
    with pytest.raises(ValueError):
        orc.forward(z, z, z, np.zeros((1, 2)), np.zeros((1, 2)), z, C0=np.zeros((1, 2, 2)))
