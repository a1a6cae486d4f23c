"""The fp64 oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_bruteforce_matches_definition_on_one_step():
    """The brute-force helper itself, on T = 1 where every term is explicit:
    y_0 = (C_0 . B_0) x_0 + a_0 (C_0 . h0) + D x_0."""
    import numpy as np
    rng = np.random.default_rng(5)
    x, Bm, Cm = pins.crandn(rng, 1, 1, 1, 2), pins.crandn(rng, 1, 1, 1, 3), pins.crandn(rng, 1, 1, 1, 3)
    h0 = pins.crandn(rng, 1, 1, 3, 2)
    dt = np.array([[[0.4]]]); A = np.array([-0.3 + 0.8j]); Dk = np.array([1.5])
    y, hT = pins.bruteforce(x, Bm, Cm, dt, A, Dk, h0)
    a = np.exp(np.log1p(np.exp(0.4)) * A[0])
    want = (Cm[0, 0, 0] @ Bm[0, 0, 0]) * x[0, 0, 0] + a * (Cm[0, 0, 0] @ h0[0, 0]) + 1.5 * x[0, 0, 0]
    assert np.allclose(y[0, 0, 0], want, rtol=1e-14, atol=1e-14)
    assert np.allclose(hT[0, 0], np.outer(Bm[0, 0, 0], x[0, 0, 0]) + a * h0[0, 0], rtol=1e-14, atol=1e-14)
